// Drives every entry point of the C ABI on the CPU, against a stub HIP
// runtime, so the library's host code (argument validation, split and
// attention planning, workspace carve-up, launch sequencing, the trace and
// the static-scratch lookup) runs under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Device pointers are fake addresses that no
// host code may dereference (a dereference faults under ASan).  Exits
// non-zero on any unexpected status.  Test infrastructure only.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "dflash2.h"

extern "C" long hc_launches();
extern "C" long hc_bad_launches();

namespace {

int g_fail = 0;

void expect(dflash2_status got, dflash2_status want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, int(got), int(want), dflash2_last_error());
    ++g_fail;
  }
}

// fake device addresses: distinct, 256-aligned, never dereferenced on the host
template <typename T>
T* dev(uintptr_t i) {
  return reinterpret_cast<T*>(uintptr_t(0x100000000000ull) + (i % 4096) * (uintptr_t(1) << 32));
}

struct Shape {
  const char* name;
  int B, bs, H, nL, nq, nkv, d, F, V, nT, Ht, Lmax, k, r, dtype, conv_group, window;
  int64_t new_rows;
};

dflash2_config config_of(const Shape& s) {
  dflash2_config c{};
  c.hidden = s.H; c.num_layers = s.nL; c.num_q_heads = s.nq; c.num_kv_heads = s.nkv; c.head_dim = s.d;
  c.ffn = s.F; c.vocab = s.V; c.num_taps = s.nT; c.tap_width = s.Ht; c.block_size = s.bs;
  c.conv_kernel_size = 2; c.selector_top_k = s.k; c.selector_rank = s.r; c.max_batch = s.B;
  c.max_context = s.Lmax; c.sliding_window = s.window; c.mask_token_id = s.V - 1; c.weight_dtype = s.dtype;
  c.conv_group_size = s.conv_group;
  c.rms_eps = 1e-6f; c.rope_theta = 1e6f; c.input_embedding_scale = 1.0f; c.output_multiplier = 1.0f;
  c.final_logit_softcapping = 0.0f;
  return c;
}

void run_shape(const Shape& s) {
  const dflash2_config c = config_of(s);
  std::vector<dflash2_layer_weights> layers(s.nL);
  uintptr_t id = 1;
  for (auto& L : layers) {
    L.conv_attn = dev<void>(id++); L.attn_norm = dev<void>(id++); L.wqkv = dev<void>(id++);
    L.wqkv_scale = dev<float>(id++); L.wo = dev<void>(id++); L.wo_scale = dev<float>(id++);
    L.conv_ffn = dev<void>(id++); L.ffn_norm = dev<void>(id++); L.w_gate_up = dev<void>(id++);
    L.w_gate_up_scale = dev<float>(id++); L.w_down = dev<void>(id++); L.w_down_scale = dev<float>(id++);
    L.dconv_attn = dev<void>(id++); L.dconv_attn_scale = dev<float>(id++);
    L.dconv_ffn = dev<void>(id++); L.dconv_ffn_scale = dev<float>(id++);
  }
  dflash2_weights w{};
  w.embed = dev<void>(id++); w.lm_head = dev<void>(id++); w.lm_head_scale = dev<float>(id++);
  w.proj = dev<void>(id++); w.proj_scale = dev<float>(id++); w.proj_norm = dev<void>(id++);
  w.final_norm = dev<void>(id++); w.sel_tl = dev<float>(id++); w.sel_tr = dev<float>(id++);
  w.layers = layers.data();
  dflash2_handle* h = nullptr;
  expect(dflash2_create(&c, &w, &h), DFLASH2_OK, s.name);
  if (!h) return;
  hipStream_t st = reinterpret_cast<hipStream_t>(uintptr_t(0x1234));
  for (int B = 1; B <= s.B; B = B < s.B ? std::min(s.B, B * 4) : s.B + 1) {
    for (int64_t rows : {int64_t(0), int64_t(B), s.new_rows}) {
      size_t ws = 0;
      expect(dflash2_workspace_size(h, B, rows, &ws), DFLASH2_OK, "workspace_size");
      auto ws_ptr = dev<void>(id++);
      // the trace records one event pair per launch
      std::vector<dflash2_trace_entry> tr(4096);
      for (auto& e : tr) {
        e.start = reinterpret_cast<hipEvent_t>(uintptr_t(0x9000));
        e.stop = reinterpret_cast<hipEvent_t>(uintptr_t(0x9001));
      }
      expect(dflash2_trace_attach(tr.data(), int32_t(tr.size())), DFLASH2_OK, "trace_attach");
      const uintptr_t p = id;
      id += 16;
      expect(dflash2_draft_block(h, st, B, dev<int32_t>(p), rows ? dev<void>(p + 1) : nullptr, dev<int32_t>(p + 2),
                                 dev<int32_t>(p + 3), rows, dev<void>(p + 4), dev<void>(p + 5), dev<int32_t>(p + 6),
                                 dev<float>(p + 7), (B & 1) ? dev<float>(p + 8) : nullptr,
                                 (B & 1) ? dev<float>(p + 9) : nullptr, ws_ptr, ws),
             DFLASH2_OK, s.name);
      const int32_t n = dflash2_trace_detach();
      if (n <= 0 || n > int32_t(tr.size())) {
        std::fprintf(stderr, "FAIL %s: %d trace entries\n", s.name, n);
        ++g_fail;
      }
      for (int32_t i = 0; i < n; ++i)
        if (tr[i].bytes < 0 || tr[i].flops < 0) {
          std::fprintf(stderr, "FAIL %s: negative trace figures at %d\n", s.name, i);
          ++g_fail;
        }
      // a workspace one byte short is rejected before any launch
      const long before = hc_launches();
      expect(dflash2_draft_block(h, st, B, dev<int32_t>(p), rows ? dev<void>(p + 1) : nullptr, dev<int32_t>(p + 2),
                                 dev<int32_t>(p + 3), rows, dev<void>(p + 4), dev<void>(p + 5), dev<int32_t>(p + 6),
                                 dev<float>(p + 7), nullptr, nullptr, ws_ptr, ws - 1),
             DFLASH2_ERR_WORKSPACE, "short workspace");
      if (hc_launches() != before) {
        std::fprintf(stderr, "FAIL %s: launches after a rejected call\n", s.name);
        ++g_fail;
      }
    }
    {
      size_t ws = 0;
      expect(dflash2_workspace_size(h, B, s.new_rows, &ws), DFLASH2_OK, "workspace_size");
      for (int dl = 0; dl < 2; ++dl)
        expect(dflash2_draft_select(h, st, B, dev<int32_t>(1), dev<void>(2), dev<int32_t>(3), dev<int32_t>(4),
                                    s.new_rows, dev<void>(5), dev<void>(6), dev<int32_t>(7), dev<float>(8),
                                    dev<int32_t>(9), dev<int32_t>(10), dl ? dev<float>(11) : nullptr,
                                    dl ? dev<float>(12) : nullptr, dev<void>(13), ws),
               DFLASH2_OK, "draft_select");
      expect(dflash2_draft_select(h, st, B, dev<int32_t>(1), dev<void>(2), dev<int32_t>(3), dev<int32_t>(4),
                                  s.new_rows, dev<void>(5), dev<void>(6), dev<int32_t>(7), dev<float>(8), nullptr,
                                  dev<int32_t>(10), nullptr, nullptr, dev<void>(13), ws),
             DFLASH2_ERR_INVALID_ARG, "draft_select null path");
    }
    expect(dflash2_select_path(h, st, B, dev<int32_t>(1), dev<int32_t>(2), dev<float>(3), dev<int32_t>(4),
                               dev<int32_t>(5), dev<float>(6), dev<float>(7)),
           DFLASH2_OK, "select_path");
    expect(dflash2_select_path_stop(h, st, B, dev<int32_t>(1), dev<int32_t>(2), dev<float>(3), 0.25f, 1, s.bs,
                                    dev<int32_t>(4), dev<int32_t>(5), dev<int32_t>(6), dev<float>(7), nullptr),
           DFLASH2_OK, "select_path_stop");
    size_t lws = 0;
    expect(dflash2_draft_losses_workspace_size(B, s.bs, s.V, &lws), DFLASH2_OK, "losses ws");
    expect(dflash2_draft_losses(h, st, B, dev<int32_t>(1), dev<int32_t>(2), dev<float>(3), dev<int32_t>(4),
                                dev<float>(5), 7.0f, 0.5f, dev<float>(6), dev<float>(7), dev<float>(8), dev<void>(9),
                                lws),
           DFLASH2_OK, "draft_losses");
  }
  expect(dflash2_workspace_size(h, s.B + 1, 0, nullptr), DFLASH2_ERR_INVALID_ARG, "null bytes");
  size_t ws = 0;
  expect(dflash2_workspace_size(h, s.B + 1, 0, &ws), DFLASH2_ERR_SHAPE, "batch > max");
  expect(dflash2_workspace_size(h, 1, (int64_t(1) << 30) + 1, &ws), DFLASH2_ERR_SHAPE, "rows > 2^30");
  dflash2_destroy(h);
}

void run_verify(int B, int bs, int V) {
  hipStream_t st = nullptr;
  size_t ws = 0, sws = 0;
  expect(dflash2_verify_workspace_size(B, bs, V, &ws), DFLASH2_OK, "verify ws");
  expect(dflash2_verify_accept(st, B, bs, V, dev<int32_t>(1), dev<float>(2), dev<int32_t>(3), dev<int32_t>(4),
                               dev<int32_t>(5), dev<void>(6), ws),
         DFLASH2_OK, "verify_accept");
  if (ws > 0)
    expect(dflash2_verify_accept(st, B, bs, V, dev<int32_t>(1), dev<float>(2), dev<int32_t>(3), dev<int32_t>(4),
                                 nullptr, dev<void>(6), ws - 1),
           DFLASH2_ERR_WORKSPACE, "verify short ws");
  const dflash2_status na = dflash2_verify_accept_noalloc(st, B, bs, V, dev<int32_t>(1), dev<float>(2),
                                                          dev<int32_t>(3), dev<int32_t>(4), nullptr);
  expect(na, int64_t(B) * bs <= 131072 ? DFLASH2_OK : DFLASH2_ERR_WORKSPACE, "verify_accept_noalloc");
  expect(dflash2_verify_sample_workspace_size(B, bs, V, &sws), DFLASH2_OK, "sample ws");
  for (float T : {0.0f, 1.0f})
    for (int tk : {0, 20})
      expect(dflash2_verify_sample(st, B, bs, V, dev<int32_t>(1), tk ? nullptr : dev<int32_t>(2),
                                   dev<float>(3), dev<float>(4), T, tk, 0.95f, dev<int32_t>(5), dev<int32_t>(6),
                                   dev<float>(7), dev<void>(8), sws),
             DFLASH2_OK, "verify_sample");
  expect(dflash2_verify_sample(st, B, bs, V, dev<int32_t>(1), nullptr, dev<float>(3), dev<float>(4), NAN, 0, 1.0f,
                               dev<int32_t>(5), dev<int32_t>(6), nullptr, dev<void>(8), sws),
         DFLASH2_ERR_INVALID_ARG, "verify_sample NaN temperature");
}

}  // namespace

int main() {
  const Shape shapes[] = {
      // name, B, bs, H, nL, nq, nkv, d, F, V, nT, Ht, Lmax, k, r, dtype, conv_group, window, new_rows
      {"tiny_fp32", 1, 8, 64, 1, 4, 4, 16, 256, 512, 2, 64, 64, 4, 8, DFLASH2_FP32, 0, 0, 32},
      {"small_bf16", 3, 8, 320, 2, 10, 2, 64, 736, 3001, 3, 192, 352, 16, 16, DFLASH2_BF16, 0, 64, 40},
      {"medium_fp8_dyn", 40, 7, 320, 2, 10, 2, 64, 768, 2500, 3, 192, 224, 8, 16, DFLASH2_FP8_E4M3, 64, 0, 200},
      {"dense27b_bf16", 1, 8, 5120, 5, 40, 8, 128, 17408, 151936, 5, 5120, 4128, 16, 64, DFLASH2_BF16, 0, 0, 8},
      {"batched_bf16", 64, 7, 4096, 1, 32, 8, 128, 14336, 131072, 3, 4096, 2080, 16, 32, DFLASH2_BF16, 0, 0, 448},
      {"longblock_bf16", 16, 16, 4096, 2, 32, 8, 128, 14336, 151936, 4, 4096, 8224, 16, 64, DFLASH2_BF16, 0, 0, 256},
      {"fp8_b256", 256, 8, 5120, 1, 40, 8, 128, 17408, 151936, 5, 5120, 2080, 16, 64, DFLASH2_FP8_E4M3, 0, 0, 2048},
      {"wide_vocab", 10, 8, 8192, 1, 2, 1, 64, 64, 270000, 1, 64, 32, 4, 8, DFLASH2_BF16, 0, 0, 16},
      {"k64_r256", 2, 8, 256, 1, 4, 1, 64, 512, 4096, 1, 256, 64, 64, 256, DFLASH2_BF16, 0, 0, 4},
  };
  for (const Shape& s : shapes) run_shape(s);
  for (int B : {1, 7, 256, 20000})
    for (int bs : {2, 8, 16}) run_verify(B, bs, B > 1000 ? 4096 : 151936);
  run_verify(70000, 4096, 3);  // 2^28 rows: grid x beyond 65535
  {
    size_t ws = 0;
    expect(dflash2_verify_workspace_size(1, 4097, 100, &ws), DFLASH2_ERR_SHAPE, "block_size 4097");
    expect(dflash2_verify_workspace_size(1 << 27, 9, 100, &ws), DFLASH2_ERR_SHAPE, "rows > 2^30");
    expect(dflash2_verify_sample_workspace_size(2, 1, 100, &ws), DFLASH2_ERR_SHAPE, "block_size 1");
    expect(dflash2_draft_losses_workspace_size(1, 8, 0, &ws), DFLASH2_ERR_SHAPE, "vocab 0");
  }
  // configurations create must reject before anything else happens
  {
    dflash2_config c = config_of(shapes[0]);
    dflash2_weights w{};
    dflash2_handle* h = nullptr;
    expect(dflash2_create(&c, &w, &h), DFLASH2_ERR_INVALID_ARG, "null weights");
    c.output_multiplier = -1.0f;
    expect(dflash2_create(&c, &w, &h), DFLASH2_ERR_INVALID_ARG, "negative multiplier");
    c = config_of(shapes[0]);
    c.num_taps = 1 << 16;
    c.tap_width = 1 << 16;
    expect(dflash2_create(&c, &w, &h), DFLASH2_ERR_UNSUPPORTED, "taps overflow int32");
    c = config_of(shapes[0]);
    c.block_size = 1;
    expect(dflash2_create(&c, &w, &h), DFLASH2_ERR_SHAPE, "block_size 1");
    c.block_size = 5000;
    c.max_context = 8192;
    expect(dflash2_create(&c, &w, &h), DFLASH2_ERR_SHAPE, "block_size 5000");
    c.block_size = 8;
    c.max_batch = 1 << 28;
    expect(dflash2_create(&c, &w, &h), DFLASH2_ERR_SHAPE, "max_batch * block_size > 2^30");
  }
  std::printf("launches %ld, bad launches %ld, failures %d\n", hc_launches(), hc_bad_launches(), g_fail);
  return (g_fail == 0 && hc_bad_launches() == 0 && hc_launches() > 0) ? 0 : 1;
}

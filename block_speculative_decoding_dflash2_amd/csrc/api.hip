// Host side of the C ABI: argument validation, work planning (split-K
// factors, attention chunking, workspace carve-up) and the launch sequence
// of one draft step.  No device memory is allocated and no call
// synchronises; everything is enqueued on the caller's stream.
#include <algorithm>
#include <cstdlib>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "dflash2.h"
#include "kernels.h"

using namespace dfl;

struct dflash2_handle {
  dflash2_config cfg;
  dflash2_weights w;
  std::vector<dflash2_layer_weights> layers;
};

namespace {

thread_local std::string g_error;

dflash2_status fail(dflash2_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

dflash2_status ok() {
  g_error.clear();
  return DFLASH2_OK;
}

// Per-thread kernel trace (see dflash2_trace_attach).
struct Trace {
  dflash2_trace_entry* entries = nullptr;
  int32_t capacity = 0, count = 0;
};
thread_local Trace g_trace;

template <typename F>
void traced(hipStream_t s, int kind, int64_t bytes, int64_t flops, F&& launch) {
  Trace& t = g_trace;
  dflash2_trace_entry* e = (t.entries && t.count < t.capacity) ? &t.entries[t.count++] : nullptr;
  if (e) {
    e->kind = kind;
    e->bytes = bytes;
    e->flops = flops;
    (void)hipEventRecord(e->start, s);
  }
  launch();
  if (e) (void)hipEventRecord(e->stop, s);
}

// Plans are a pure function of the shapes (not of the device), so results
// and workspace sizes do not depend on which GPU runs them.
constexpr int kTargetBlocks = 512;  // 2 blocks of 4 waves per CU on 256 CUs
constexpr int kStreamBlockOverhead = 256;  // fixed cost of one weight-streaming block, in k
constexpr int64_t kStreamMaxRowBytes = 3072;  // longest per-block stream of one weight row
constexpr size_t kAlign = 256;
// Row bounds shared by every entry point: block_size <= 4096 (the greedy
// verifier keeps a block's argmaxes in LDS) and batch * block_size <= 2^30
// rows (row indices are 32-bit and rows are grid x-blocks).
constexpr int32_t kMaxBlockSize = 4096;
constexpr int64_t kMaxRows = int64_t(1) << 30;
bool rows_ok(int32_t batch, int32_t block_size) {
  return batch >= 1 && block_size >= 2 && block_size <= kMaxBlockSize && int64_t(batch) * block_size <= kMaxRows;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
// The kernels read weights, activations and caches 16 bytes at a time.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int act_bytes(const dflash2_config& c) { return c.weight_dtype == DFLASH2_FP32 ? 4 : 2; }
int weight_bytes(const dflash2_config& c) {
  return c.weight_dtype == DFLASH2_FP32 ? 4 : (c.weight_dtype == DFLASH2_BF16 ? 2 : 1);
}

struct Split {
  int splits = 1, k_split = 0;
  int tile_rows = 0;  // LDS-tiled GEMM: activation rows per block tile
};

Split plan_split(int dtype, int M, int N, int K, int groups = 1) {
  Split s;
  if (gemm_tiled_ok(dtype, M, K)) {
    // compute-bound tiles: the block tile (256 or 128 activation rows) and
    // split count with the shortest estimated time, counting waves of
    // resident tiles (256 CUs x tiles per CU), each costing its k range plus
    // a fixed prologue/epilogue of about 512 k at ~1.2 PF/s of 256-row tiles
    // (fp8 128-row tiles, two per CU, measured up to ~10% slower per flop
    // than 256-row tiles with three stage buffers, fp8 192-row tiles taken
    // as 4% slower; bf16 128-row tiles, one per CU, ~20% slower), plus the
    // float32 partial
    // sums every split writes and its consumer reads back (8 bytes per
    // output per split at ~5 TB/s); ties go to fewer splits and larger
    // tiles, at most 16 splits (a 60 x 4096 x 16384 projection of the
    // long-block workload ran 51 us on 8 splits, 42 us on 16: 16 column tiles
    // need 16 splits to occupy the 256 CUs).
    int max_splits = 16;
    if (const char* env = std::getenv("DFLASH2_TILED_MAX_SPLITS")) {
      const int v = std::atoi(env);
      if (v >= 1 && v <= 16) max_splits = v;
    }
    double best_cost = 1e300;
    for (int bm : {256, 192, 128}) {
      const TiledShape sh = tiled_shape(dtype, M, bm);
      if (sh.bm != bm) continue;
      const int64_t tiles = cdiv(M, sh.bm) * cdiv(N, 256) * groups;
      const int64_t slots = 256 * int64_t(sh.per_cu);
      const double eff = sh.bm == 256 ? 1.0 : (sh.bm == 192 ? 1.04 : (sh.per_cu == 2 ? 1.1 : 1.2));
      const double us_per_k = 2.0 * 256.0 * sh.bm * sh.per_cu / 4.7e6 * eff;  // one tile, per k, in us
      for (int S = 1; S <= max_splits; ++S) {
        const int64_t ks = cdiv(cdiv(K, S), 64) * 64;
        if (cdiv(K, ks) != S) continue;
        const double cost = double(cdiv(tiles * S, slots)) * double(ks + 512) * us_per_k +
                            8.0 * S * double(M) * N * groups / 5e6;
        if (cost < best_cost * 0.97) {
          best_cost = cost;
          s.splits = S;
          s.tile_rows = sh.bm;
        }
      }
    }
    s.k_split = int(cdiv(cdiv(K, s.splits), 64) * 64);
    s.splits = int(cdiv(K, s.k_split));
    return s;
  }
  const int mtile = M <= 16 ? 16 : (M <= 32 ? 32 : 64);
  const int64_t blocks = cdiv(N, gemm_rows_per_block(dtype, M)) * cdiv(M, mtile) * groups;
  int S = 1;
  if (M <= 64) {
    // weight streaming: the shortest makespan over waves of kTargetBlocks
    // resident blocks, each costing its k range plus a fixed prologue /
    // epilogue of about kStreamBlockOverhead k; ties go to fewer splits.
    // (Rounding the split count up to fill the slots made grids of 520-560
    // blocks, whose second wave of 8-48 blocks doubled the kernel's time.)
    int overhead = kStreamBlockOverhead, target = kTargetBlocks;
    if (const char* env = std::getenv("DFLASH2_STREAM_BLOCK_OVERHEAD")) {
      const int v = std::atoi(env);
      if (v >= 0 && v <= 65536) overhead = v;
    }
    if (const char* env = std::getenv("DFLASH2_STREAM_TARGET_BLOCKS")) {
      const int v = std::atoi(env);
      if (v >= 64 && v <= 8192) target = v;
    }
    // Each block's stream is also kept to at most kStreamMaxRowBytes of every
    // weight row: the 5120 x 25600 feature projection measured 55 us with 480
    // blocks of 4288 bytes per row and 43 us with 1000 blocks of 2048 bytes
    // (both by this cost model's count the first was cheaper).
    int64_t max_row_bytes = kStreamMaxRowBytes;
    if (const char* env = std::getenv("DFLASH2_STREAM_MAX_ROW_BYTES")) {
      const int v = std::atoi(env);
      if (v >= 256 && v <= (1 << 20)) max_row_bytes = v;
    }
    const int wb = dtype == 0 ? 4 : (dtype == 1 ? 2 : 1);
    const int max_s = std::max(1, std::min(64, K / 256));
    double best_cost = 1e300;
    bool best_capped = false;
    for (int c = 1; c <= max_s; ++c) {
      const int64_t ks = cdiv(cdiv(K, c), 32) * 32;
      if (cdiv(K, ks) != c) continue;
      const bool capped = ks * wb <= max_row_bytes;
      const double cost = double(cdiv(blocks * c, target)) * double(ks + overhead);
      if ((capped && !best_capped) || (capped == best_capped && cost < best_cost * 0.999)) {
        best_cost = cost;
        best_capped = capped;
        S = c;
      }
    }
  }
  s.k_split = int(cdiv(cdiv(K, S), 32) * 32);
  s.splits = int(cdiv(K, s.k_split));
  return s;
}

struct AttnPlan {
  int chunk = 128, nchunks = 1, qgroups = 1, qs = 1;
};

// Chunks of whole LDS sub-chunks; enough sub-chunks per block that the grid
// is about kTargetBlocks blocks (fewer, larger chunks mean fewer partials).
AttnPlan plan_attn(const dflash2_config& c, int B) {
  AttnPlan a;
  const int grp = c.num_q_heads / c.num_kv_heads;
  a.qs = c.block_size * grp;
  a.qgroups = int(cdiv(a.qs, 64));
  const int kt = attn_sub_chunk(c.weight_dtype == DFLASH2_FP32, c.head_dim);
  const int64_t subs = cdiv(c.max_context, kt);
  const int64_t heads = int64_t(B) * c.num_kv_heads * a.qgroups;
  int64_t target = kTargetBlocks;
  if (const char* env = std::getenv("DFLASH2_ATTN_TARGET_BLOCKS")) {
    const int v = std::atoi(env);
    if (v >= 64 && v <= 65536) target = v;
  }
  // at least three sub-chunks per block: with fewer (8 heads at batch 1, the
  // 27B-class workload) the partials and their merge cost more than the
  // extra blocks gain (attention + merge 101 -> 94 us per step)
  const int64_t per_block = std::max<int64_t>(std::min<int64_t>(3, subs), cdiv(heads * subs, target));
  a.chunk = int(per_block * kt);
  a.nchunks = int(cdiv(c.max_context, a.chunk));
  return a;
}

struct Plan {
  int B, M, Mh, Mn;
  Split proj, kv, qkv, o, gu, down, dconv;
  AttnPlan attn;
  int groups;
  size_t off_h0, off_h1, off_n, off_sumsq, off_q, off_o, off_a, off_parts, off_attn_o, off_attn_ml,
      off_cand, off_cand2, off_hpre;
  size_t total;
};

Plan make_plan(const dflash2_config& c, int B, int64_t Mn) {
  Plan p;
  p.B = B;
  p.M = B * c.block_size;
  p.Mh = B * (c.block_size - 1);
  p.Mn = int(Mn);
  const int H = c.hidden, qd = c.num_q_heads * c.head_dim, kvd = 2 * c.num_kv_heads * c.head_dim;
  const int qkvd = qd + kvd, F = c.ffn, dt = c.weight_dtype;
  p.proj = plan_split(dt, std::max(p.Mn, 1), H, c.num_taps * c.tap_width);
  p.kv = plan_split(dt, std::max(p.Mn, 1), kvd, H, std::min(c.num_layers, kMaxGroups));
  p.qkv = plan_split(dt, p.M, qkvd, H);
  p.o = plan_split(dt, p.M, H, qd);
  p.gu = plan_split(dt, p.M, 2 * F, H);
  p.down = plan_split(dt, p.M, H, F);
  const int gk = c.conv_group_size > 0 ? H / c.conv_group_size * c.conv_kernel_size : 0;
  p.dconv = gk > 0 ? plan_split(dt, p.M, gk, H) : Split{1, H};
  p.attn = plan_attn(c, B);
  p.groups = int(cdiv(c.vocab, kLmGroupIds));
  const size_t ab = act_bytes(c);
  size_t parts = 0;
  auto upd = [&](size_t v) { parts = std::max(parts, v); };
  if (p.Mn > 0) {
    upd(size_t(p.proj.splits) * p.Mn * H);
    upd(size_t(c.num_layers) * p.kv.splits * p.Mn * kvd);
  }
  upd(size_t(p.qkv.splits) * p.M * qkvd);
  upd(size_t(p.o.splits) * p.M * H);
  upd(size_t(p.gu.splits) * p.M * 2 * F);
  upd(size_t(p.down.splits) * p.M * H);
  if (gk > 0) upd(size_t(p.dconv.splits) * p.M * gk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  p.off_h0 = take(size_t(p.M) * H * 4);
  p.off_h1 = take(size_t(p.M) * H * 4);
  p.off_n = take(size_t(std::max(p.M, p.Mn)) * H * ab);
  p.off_sumsq = take(size_t(std::max(p.M, p.Mn)) * norm_col_blocks(H) * 4);
  p.off_q = take(size_t(p.M) * qd * ab);
  p.off_o = take(size_t(p.M) * qd * ab);
  p.off_a = take(size_t(p.M) * F * ab);
  p.off_parts = take(parts * 4);
  const size_t attn_rows = size_t(B) * c.num_kv_heads * p.attn.nchunks * p.attn.qs;
  p.off_attn_o = take(attn_rows * c.head_dim * 4);
  p.off_attn_ml = take(attn_rows * 2 * 4);
  // candidate lists: the weight-streaming lm_head writes groups x k keys per
  // row, the tiled one at most groups lists of 16
  p.off_cand = take(size_t(p.Mh) * p.groups * std::max(c.selector_top_k, 16) * 8);
  // their first fold (k <= 16, more than 256 lists per row): 16 keys per 64 lists
  p.off_cand2 = take(size_t(p.Mh) * topk_premerge_lists(p.groups) * 16 * 8);
  // dynamic convolution: each conv site's input rows, float32
  p.off_hpre = gk > 0 ? take(size_t(p.M) * H * 4) : 0;
  p.total = off;
  return p;
}

dflash2_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DFLASH2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DFLASH2_OK;
}

const void* byte_offset(const void* p, int64_t bytes) {
  return static_cast<const char*>(p) + bytes;
}

constexpr size_t kSelectLds = 156 * 1024;  // one window covers every position at the configs here
dflash2_status select_impl(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                           const int32_t* anchor_ids, const int32_t* topk_ids, const float* topk_vals,
                           int32_t* path_idx, int32_t* draft_tokens, float* path_score, float* debug_pair,
                           float p_min, int32_t n_min, int32_t n_max, int32_t* draft_lens,
                           float* path_conf, const char* name);

}  // namespace

extern "C" {

const char* dflash2_last_error(void) { return g_error.c_str(); }

dflash2_status dflash2_trace_attach(dflash2_trace_entry* entries, int32_t capacity) {
  if (capacity < 0 || (capacity > 0 && !entries))
    return fail(DFLASH2_ERR_INVALID_ARG, "trace_attach: bad entries/capacity");
  g_trace.entries = entries;
  g_trace.capacity = capacity;
  g_trace.count = 0;
  return ok();
}

int32_t dflash2_trace_detach(void) {
  const int32_t n = g_trace.count;
  g_trace = Trace();
  return n;
}

dflash2_status dflash2_create(const dflash2_config* config, const dflash2_weights* weights,
                              dflash2_handle** out) {
  if (!config || !weights || !out) return fail(DFLASH2_ERR_INVALID_ARG, "create: null argument");
  *out = nullptr;
  const dflash2_config& c = *config;
  if (c.hidden <= 0 || c.num_layers <= 0 || c.num_q_heads <= 0 || c.num_kv_heads <= 0 ||
      c.head_dim <= 0 || c.ffn <= 0 || c.vocab <= 0 || c.num_taps <= 0 || c.tap_width <= 0 ||
      c.max_batch <= 0 || c.max_context <= 0 || c.sliding_window < 0)
    return fail(DFLASH2_ERR_INVALID_ARG, "create: sizes must be positive");
  if (c.weight_dtype < DFLASH2_FP32 || c.weight_dtype > DFLASH2_FP8_E4M3)
    return fail(DFLASH2_ERR_INVALID_ARG, "create: unknown weight_dtype %d", c.weight_dtype);
  if (!rows_ok(c.max_batch, c.block_size))
    return fail(DFLASH2_ERR_SHAPE, "create: block_size %d outside 2..4096 or max_batch * block_size > 2^30",
                c.block_size);
  if (c.num_q_heads % c.num_kv_heads)
    return fail(DFLASH2_ERR_SHAPE, "create: num_q_heads %d not a multiple of num_kv_heads %d",
                c.num_q_heads, c.num_kv_heads);
  if (c.conv_kernel_size < 1 || c.conv_kernel_size > c.block_size)
    return fail(DFLASH2_ERR_SHAPE, "create: conv_kernel_size %d outside 1..block_size",
                c.conv_kernel_size);
  if (c.conv_group_size < 0 || (c.conv_group_size > 0 && c.hidden % c.conv_group_size))
    return fail(DFLASH2_ERR_SHAPE, "create: conv_group_size %d must be 0 or divide hidden %d",
                c.conv_group_size, c.hidden);
  if (c.selector_top_k < 1 || c.selector_top_k > 64 || c.selector_top_k > c.vocab)
    return fail(DFLASH2_ERR_SHAPE, "create: selector_top_k %d outside 1..min(64, vocab)",
                c.selector_top_k);
  if (c.selector_rank < 1 || c.selector_rank > 256)
    return fail(DFLASH2_ERR_SHAPE, "create: selector_rank %d outside 1..256", c.selector_rank);
  if (c.mask_token_id < 0 || c.mask_token_id >= c.vocab)
    return fail(DFLASH2_ERR_SHAPE, "create: mask_token_id %d outside [0, vocab)", c.mask_token_id);
  if (c.max_context < c.block_size)
    return fail(DFLASH2_ERR_SHAPE, "create: max_context %d < block_size", c.max_context);
  if (!(c.rms_eps >= 0.f) || !std::isfinite(c.rms_eps) || !(c.rope_theta > 0.f) ||
      !std::isfinite(c.rope_theta) || !(c.final_logit_softcapping >= 0.f) ||
      !std::isfinite(c.final_logit_softcapping))
    return fail(DFLASH2_ERR_INVALID_ARG, "create: bad rms_eps / rope_theta / softcap");
  // Top-k ranks the raw logits and the transform is applied to the k kept
  // values, which is the top-k of the transformed logits only while the
  // transform is strictly increasing: the multiplier must be positive.
  if (!(c.output_multiplier > 0.f) || !std::isfinite(c.output_multiplier))
    return fail(DFLASH2_ERR_INVALID_ARG, "create: output_multiplier %g must be finite and > 0",
                double(c.output_multiplier));
  if (!std::isfinite(c.input_embedding_scale))
    return fail(DFLASH2_ERR_INVALID_ARG, "create: input_embedding_scale is not finite");
  if (!attn_supported(c.head_dim))
    return fail(DFLASH2_ERR_UNSUPPORTED, "create: head_dim %d not in {16, 32, 64, 128, 256}",
                c.head_dim);
  // The GEMMs address a tile of at most 128 rows with 32-bit byte offsets
  // from a 64-bit tile base: every contraction length stays <= 2^20.
  constexpr int64_t kMaxContraction = int64_t(1) << 20;
  const int64_t qd = int64_t(c.num_q_heads) * c.head_dim;
  const int64_t kp = int64_t(c.num_taps) * c.tap_width;
  if (c.ffn > kMaxContraction || qd > kMaxContraction || kp > kMaxContraction)
    return fail(DFLASH2_ERR_UNSUPPORTED,
                "create: ffn, nq*head_dim and num_taps*tap_width must be <= 1048576");
  if (c.hidden % 32 || c.ffn % 32 || qd % 32 || kp % 32)
    return fail(DFLASH2_ERR_UNSUPPORTED,
                "create: hidden, ffn, nq*head_dim and num_taps*tap_width must be multiples of 32");
  if (c.hidden > 16384) return fail(DFLASH2_ERR_UNSUPPORTED, "create: hidden > 16384");
  if (c.max_context % 8)
    return fail(DFLASH2_ERR_UNSUPPORTED, "create: max_context must be a multiple of 8");
  if (select_window(c.selector_top_k, c.selector_rank, c.block_size - 1, kSelectLds) < 1)
    return fail(DFLASH2_ERR_UNSUPPORTED, "create: selector_top_k * selector_rank too large");
  const dflash2_weights& w = *weights;
  if (!w.embed || !w.lm_head || !w.proj || !w.proj_norm || !w.final_norm || !w.sel_tl ||
      !w.sel_tr || !w.layers)
    return fail(DFLASH2_ERR_INVALID_ARG, "create: null weight pointer");
  const bool fp8 = c.weight_dtype == DFLASH2_FP8_E4M3;
  if (fp8 && (!w.lm_head_scale || !w.proj_scale))
    return fail(DFLASH2_ERR_INVALID_ARG, "create: fp8 weights need scales");
  for (const void* q : {w.embed, w.lm_head, static_cast<const void*>(w.lm_head_scale), w.proj,
                        static_cast<const void*>(w.proj_scale), w.proj_norm, w.final_norm,
                        static_cast<const void*>(w.sel_tl), static_cast<const void*>(w.sel_tr)})
    if (!aligned16(q)) return fail(DFLASH2_ERR_INVALID_ARG, "create: weight pointers must be 16-byte aligned");
  for (int l = 0; l < c.num_layers; ++l) {
    const dflash2_layer_weights& L = w.layers[l];
    const bool dyn = c.conv_group_size > 0;
    if (!L.attn_norm || !L.wqkv || !L.wo || !L.ffn_norm || !L.w_gate_up || !L.w_down ||
        (!dyn && (!L.conv_attn || !L.conv_ffn)) || (dyn && (!L.dconv_attn || !L.dconv_ffn)))
      return fail(DFLASH2_ERR_INVALID_ARG, "create: null weight pointer in layer %d", l);
    if (fp8 && (!L.wqkv_scale || !L.wo_scale || !L.w_gate_up_scale || !L.w_down_scale ||
                (dyn && (!L.dconv_attn_scale || !L.dconv_ffn_scale))))
      return fail(DFLASH2_ERR_INVALID_ARG, "create: fp8 weights need scales (layer %d)", l);
    for (const void* q : {L.attn_norm, L.wqkv, static_cast<const void*>(L.wqkv_scale), L.wo,
                          static_cast<const void*>(L.wo_scale), L.ffn_norm, L.w_gate_up,
                          static_cast<const void*>(L.w_gate_up_scale), L.w_down,
                          static_cast<const void*>(L.w_down_scale), L.conv_attn, L.conv_ffn, L.dconv_attn,
                          static_cast<const void*>(L.dconv_attn_scale), L.dconv_ffn,
                          static_cast<const void*>(L.dconv_ffn_scale)})
      if (!aligned16(q))
        return fail(DFLASH2_ERR_INVALID_ARG, "create: weight pointers must be 16-byte aligned (layer %d)", l);
  }
  dflash2_handle* h = new dflash2_handle;
  h->cfg = c;
  h->w = w;
  h->layers.assign(w.layers, w.layers + c.num_layers);
  h->w.layers = h->layers.data();
  *out = h;
  return ok();
}

void dflash2_destroy(dflash2_handle* handle) { delete handle; }

dflash2_status dflash2_workspace_size(const dflash2_handle* handle, int32_t batch,
                                      int64_t max_new_rows, size_t* bytes) {
  if (!handle || !bytes) return fail(DFLASH2_ERR_INVALID_ARG, "workspace_size: null argument");
  if (batch < 1 || batch > handle->cfg.max_batch)
    return fail(DFLASH2_ERR_SHAPE, "workspace_size: batch %d outside 1..max_batch", batch);
  if (max_new_rows < 0 || max_new_rows > int64_t(1) << 30)
    return fail(DFLASH2_ERR_SHAPE, "workspace_size: bad max_new_rows");
  *bytes = make_plan(handle->cfg, batch, max_new_rows).total;
  return ok();
}

// Steps 1-3, and with path_idx non-null step 4 too (the candidate merge then
// runs inside the selector's kernel when k <= 16).
static dflash2_status draft_impl(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                 const int32_t* anchor_ids, const void* new_taps,
                                 const int32_t* new_offsets, const int32_t* ctx_lens,
                                 int64_t max_new_rows, void* k_cache, void* v_cache,
                                 int32_t* topk_ids, float* topk_vals, float* debug_logits,
                                 float* debug_hidden, void* workspace, size_t workspace_bytes,
                                 int32_t* path_idx, int32_t* draft_tokens, float* path_score) {
  if (!handle) return fail(DFLASH2_ERR_INVALID_ARG, "draft_block: null handle");
  if (path_idx && !draft_tokens) return fail(DFLASH2_ERR_INVALID_ARG, "draft_select: null draft_tokens");
  const dflash2_config& c = handle->cfg;
  if (batch < 1 || batch > c.max_batch)
    return fail(DFLASH2_ERR_SHAPE, "draft_block: batch %d outside 1..max_batch %d", batch, c.max_batch);
  if (max_new_rows < 0 || max_new_rows > int64_t(1) << 30)
    return fail(DFLASH2_ERR_SHAPE, "draft_block: bad max_new_rows");
  if (!anchor_ids || !new_offsets || !ctx_lens || !k_cache || !v_cache || !topk_ids || !topk_vals ||
      (max_new_rows > 0 && !new_taps))
    return fail(DFLASH2_ERR_INVALID_ARG, "draft_block: null pointer argument");
  if (!aligned16(new_taps) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(debug_logits) ||
      !aligned16(debug_hidden))
    return fail(DFLASH2_ERR_INVALID_ARG,
                "draft_block: new_taps, the caches and the debug outputs must be 16-byte aligned");
  const Plan P = make_plan(c, batch, max_new_rows);
  if (!workspace || workspace_bytes < P.total || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return fail(DFLASH2_ERR_WORKSPACE, "draft_block: workspace needs %zu bytes, 256-aligned", P.total);

  const bool f32 = c.weight_dtype == DFLASH2_FP32;
  const int dt = c.weight_dtype;
  const int H = c.hidden, nq = c.num_q_heads, nkv = c.num_kv_heads, d = c.head_dim, F = c.ffn;
  const int qd = nq * d, kvd = 2 * nkv * d, qkvd = qd + kvd, bs = c.block_size;
  const int wb = weight_bytes(c);
  char* ws = static_cast<char*>(workspace);
  float* h0 = reinterpret_cast<float*>(ws + P.off_h0);
  float* h1 = reinterpret_cast<float*>(ws + P.off_h1);
  void* nbuf = ws + P.off_n;
  float* sumsq = reinterpret_cast<float*>(ws + P.off_sumsq);
  // RMSNorm factor of the rows last written by norm(): applied by the next GEMM
  const RowScale normed{sumsq, norm_col_blocks(H), 1.0f / float(H), c.rms_eps};
  const RowScale plain{nullptr, 0, 0.f, 0.f};
  void* qbuf = ws + P.off_q;
  void* obuf = ws + P.off_o;
  void* abuf = ws + P.off_a;
  float* parts = reinterpret_cast<float*>(ws + P.off_parts);
  const int64_t cache_layer = int64_t(c.max_batch) * nkv * c.max_context * d;
  const int ab = act_bytes(c);
  char* kc = static_cast<char*>(k_cache);
  char* vc = static_cast<char*>(v_cache);
  dflash2_status st;

  // returns whether `epi` was applied inside the GEMM (else the caller runs
  // the consumer kernel on the partial sums)
  auto gemm = [&](const void* X, int64_t ldx, const void* W, const float* scale, int M,
                  const int32_t* M_dev, int N, int K, const Split& sp, float* out, const RowScale& rs,
                  const GemmEpi* epi = nullptr) {
    GemmArgs a{};
    a.rs = rs;
    if (epi) a.epi = *epi;
    a.X = X; a.ldx = ldx; a.W = W; a.ldw = K; a.scale = scale;
    a.P = out; a.ldp = N; a.split_stride = int64_t(M) * N;
    a.M = M; a.N = N; a.K = K; a.M_dev = M_dev;
    a.splits = sp.splits; a.k_split = sp.k_split; a.groups = 1; a.tile_rows = sp.tile_rows;
    const int64_t bytes = int64_t(N) * K * wb + (scale ? int64_t(N) * 4 : 0) + int64_t(M) * K * ab +
                          int64_t(M) * N * 4;
    const bool fused = epi && gemm_epi_fusable(dt, a);
    traced(stream, DFLASH2_K_GEMM, bytes, 2 * int64_t(M) * N * K, [&] { launch_gemm(dt, a, stream); });
    return fused;
  };
  const int G = c.conv_group_size;
  const int GK = G > 0 ? H / G * c.conv_kernel_size : 0;
  float* hpre = G > 0 ? reinterpret_cast<float*>(ws + P.off_hpre) : nullptr;
  auto norm = [&](int rows, const int32_t* rows_dev, int nbs, const void* embed, const float* base,
                  const float* prt, const Split* sp, int64_t pstride, const void* conv,
                  const void* gain, float* h_out, void* n_out, int t_first, const float* dtaps = nullptr) {
    NormArgs a{};
    if (dtaps) {
      a.dtaps = dtaps; a.dsplits = P.dconv.splits; a.dstride = int64_t(rows) * GK; a.dgk = GK; a.dgroup = G;
    }
    a.H = H; a.rows = rows; a.rows_dev = rows_dev; a.bs = nbs;
    a.embed = embed; a.anchors = anchor_ids; a.mask_id = c.mask_token_id; a.vocab = c.vocab;
    a.emb_scale = c.input_embedding_scale;
    a.base = base; a.parts = prt; a.splits = sp ? sp->splits : 0; a.split_stride = pstride; a.ldp = H;
    a.conv = conv; a.conv_k = c.conv_kernel_size; a.gain = gain;
    a.h_out = h_out; a.n_out = n_out; a.sumsq = sumsq; a.t_first = t_first;
    const int64_t in_rows = int64_t(rows) * H * ((embed ? ab : 0) + (base ? 4 : 0) + 4 * a.splits) +
                            (dtaps ? int64_t(rows) * GK * 4 * a.dsplits : 0);
    const int64_t out_rows = int64_t(rows) * H * ((h_out ? 4 : 0) + ab);
    traced(stream, DFLASH2_K_NORM, in_rows + out_rows, 0, [&] { launch_norm(f32, a, stream); });
  };

  // Residual update + in-block convolution + RMSNorm of the block rows.  With
  // dynamic taps (conv_group_size > 0) the conv input is materialised first
  // (float32 for the conv, the activation dtype for the tap GEMM), the taps of
  // every slot are one GEMM against W_dconv, and the conv pass reads them.
  auto conv_norm = [&](const void* embed, const float* base, const float* prt, const Split* sp,
                       int64_t pstride, const void* conv, const void* dconv, const float* dscale,
                       const void* gain, float* h_out) {
    if (G == 0) {
      norm(P.M, nullptr, bs, embed, base, prt, sp, pstride, conv, gain, h_out, nbuf, 0);
      return;
    }
    norm(P.M, nullptr, bs, embed, base, prt, sp, pstride, nullptr, nullptr, hpre, nbuf, 0);
    gemm(nbuf, H, dconv, dscale, P.M, nullptr, GK, H, P.dconv, parts, plain);
    norm(P.M, nullptr, bs, nullptr, hpre, nullptr, nullptr, 0, nullptr, gain, h_out, nbuf, 0, parts);
  };

  // ---- 1. context append -------------------------------------------------
  if (P.Mn > 0) {
    const int Kp = c.num_taps * c.tap_width;
    const int32_t* rows_dev = new_offsets + batch;
    gemm(new_taps, Kp, handle->w.proj, handle->w.proj_scale, P.Mn, rows_dev, H, Kp, P.proj, parts, plain);
    norm(P.Mn, rows_dev, 1, nullptr, nullptr, parts, &P.proj, int64_t(P.Mn) * H, nullptr,
         handle->w.proj_norm, nullptr, nbuf, 0);
    // every layer's K/V rows of W_qkv, up to kMaxGroups layers per launch
    const int64_t lstride = int64_t(P.kv.splits) * P.Mn * kvd;
    for (int l0 = 0; l0 < c.num_layers; l0 += kMaxGroups) {
      const int ng = std::min(kMaxGroups, c.num_layers - l0);
      GemmArgs a{};
      a.rs = normed;
      a.X = nbuf; a.ldx = H; a.ldw = H;
      a.P = parts + l0 * lstride; a.ldp = kvd; a.split_stride = int64_t(P.Mn) * kvd;
      a.M = P.Mn; a.N = kvd; a.K = H; a.M_dev = rows_dev;
      a.splits = P.kv.splits; a.k_split = P.kv.k_split; a.tile_rows = P.kv.tile_rows;
      a.groups = ng; a.group_stride = lstride;
      for (int g = 0; g < ng; ++g) {
        const dflash2_layer_weights& L = handle->layers[l0 + g];
        a.Wg[g] = byte_offset(L.wqkv, int64_t(qd) * H * wb);
        a.Sg[g] = (dt == DFLASH2_FP8_E4M3 && L.wqkv_scale) ? L.wqkv_scale + qd : nullptr;
      }
      a.W = a.Wg[0]; a.scale = a.Sg[0];
      const int64_t bytes = ng * (int64_t(kvd) * H * wb + (a.Sg[0] ? int64_t(kvd) * 4 : 0) +
                                  int64_t(P.Mn) * kvd * 4) + int64_t(P.Mn) * H * ab;
      traced(stream, DFLASH2_K_GEMM, bytes, 2 * int64_t(ng) * P.Mn * kvd * H,
             [&] { launch_gemm(dt, a, stream); });
    }
    KvAppendArgs ka{};
    ka.parts = parts; ka.splits = P.kv.splits; ka.split_stride = int64_t(P.Mn) * kvd; ka.ldp = kvd;
    ka.layer_stride = lstride; ka.offsets = new_offsets; ka.ctx_lens = ctx_lens;
    ka.B = batch; ka.Mn = P.Mn; ka.nkv = nkv; ka.d = d; ka.Lmax = c.max_context; ka.nL = c.num_layers;
    ka.cache_layer_stride = cache_layer; ka.theta = c.rope_theta;
    ka.k_cache = k_cache; ka.v_cache = v_cache;
    traced(stream, DFLASH2_K_KV_APPEND, int64_t(P.Mn) * c.num_layers * kvd * (4 * P.kv.splits + ab), 0,
           [&] { launch_kv_append(f32, ka, stream); });
    if ((st = check_launch("draft_block/append")) != DFLASH2_OK) return st;
  }

  // ---- 2. block forward --------------------------------------------------
  const dflash2_layer_weights& L0 = handle->layers[0];
  conv_norm(handle->w.embed, nullptr, nullptr, nullptr, 0, L0.conv_attn, L0.dconv_attn,
            dt == DFLASH2_FP8_E4M3 ? L0.dconv_attn_scale : nullptr, L0.attn_norm, h0);
  for (int l = 0; l < c.num_layers; ++l) {
    const dflash2_layer_weights& L = handle->layers[l];
    const bool fp8 = dt == DFLASH2_FP8_E4M3;
    void* kl = kc + l * cache_layer * ab;
    void* vl = vc + l * cache_layer * ab;
    GemmEpi qe{};
    qe.kind = EPI_QKV;
    qe.ctx_lens = ctx_lens; qe.bs = bs; qe.nq = nq; qe.nkv = nkv; qe.d = d; qe.Lmax = c.max_context;
    qe.theta = c.rope_theta; qe.q_out = qbuf; qe.k_layer = kl; qe.v_layer = vl;
    if (!gemm(nbuf, H, L.wqkv, fp8 ? L.wqkv_scale : nullptr, P.M, nullptr, qkvd, H, P.qkv, parts, normed, &qe)) {
      QkvEpiArgs qa{};
      qa.parts = parts; qa.splits = P.qkv.splits; qa.split_stride = int64_t(P.M) * qkvd; qa.ldp = qkvd;
      qa.ctx_lens = ctx_lens; qa.M = P.M; qa.bs = bs; qa.nq = nq; qa.nkv = nkv; qa.d = d;
      qa.Lmax = c.max_context; qa.theta = c.rope_theta; qa.q_out = qbuf; qa.k_layer = kl; qa.v_layer = vl;
      traced(stream, DFLASH2_K_QKV_EPILOGUE, int64_t(P.M) * qkvd * (4 * P.qkv.splits + ab), 0,
             [&] { launch_qkv_epilogue(f32, qa, stream); });
    }

    AttnArgs aa{};
    aa.q = qbuf; aa.k_layer = kl; aa.v_layer = vl; aa.ctx_lens = ctx_lens;
    aa.B = batch; aa.bs = bs; aa.nq = nq; aa.nkv = nkv; aa.d = d; aa.Lmax = c.max_context;
    aa.window = c.sliding_window; aa.chunk_keys = P.attn.chunk; aa.nchunks = P.attn.nchunks;
    aa.qgroups = P.attn.qgroups;
    aa.part_o = reinterpret_cast<float*>(ws + P.off_attn_o);
    aa.part_ml = reinterpret_cast<float*>(ws + P.off_attn_ml);
    aa.scale_log2 = float(1.4426950408889634 / std::sqrt(double(d)));
    aa.o = obuf;  // used only with one chunk: the kernel then writes the output itself
    const bool one_chunk = P.attn.nchunks == 1;
    // keys/values of every sequence at the host-side bound max_context
    const int64_t kv_bytes = int64_t(batch) * nkv * c.max_context * d * 2 * ab;
    traced(stream, DFLASH2_K_ATTENTION, kv_bytes + int64_t(P.M) * qd * ab * (one_chunk ? 2 : 1),
           4 * int64_t(P.M) * qd * c.max_context, [&] { launch_attention(f32, aa, stream); });
    if (!one_chunk) {
      AttnCombineArgs ca{};
      ca.part_o = aa.part_o; ca.part_ml = aa.part_ml; ca.ctx_lens = ctx_lens;
      ca.B = batch; ca.bs = bs; ca.nq = nq; ca.nkv = nkv; ca.d = d; ca.Lmax = c.max_context;
      ca.window = c.sliding_window; ca.chunk_keys = P.attn.chunk; ca.nchunks = P.attn.nchunks;
      ca.o = obuf;
      traced(stream, DFLASH2_K_ATTN_COMBINE, int64_t(P.M) * qd * ab, 0,
             [&] { launch_attn_combine(f32, ca, stream); });
    }

    gemm(obuf, qd, L.wo, fp8 ? L.wo_scale : nullptr, P.M, nullptr, H, qd, P.o, parts, plain);
    conv_norm(nullptr, h0, parts, &P.o, int64_t(P.M) * H, L.conv_ffn, L.dconv_ffn,
              fp8 ? L.dconv_ffn_scale : nullptr, L.ffn_norm, h1);
    GemmEpi se{};
    se.kind = EPI_SWIGLU;
    se.act_out = abuf; se.F = F;
    if (!gemm(nbuf, H, L.w_gate_up, fp8 ? L.w_gate_up_scale : nullptr, P.M, nullptr, 2 * F, H, P.gu, parts,
              normed, &se)) {
      SwigluArgs sa{};
      sa.parts = parts; sa.splits = P.gu.splits; sa.split_stride = int64_t(P.M) * 2 * F; sa.ldp = 2 * F;
      sa.M = P.M; sa.F = F; sa.out = abuf;
      traced(stream, DFLASH2_K_SWIGLU, int64_t(P.M) * F * (8 * P.gu.splits + ab), 0,
             [&] { launch_swiglu(f32, sa, stream); });
    }
    gemm(abuf, F, L.w_down, fp8 ? L.w_down_scale : nullptr, P.M, nullptr, H, F, P.down, parts, plain);
    if (l + 1 < c.num_layers) {
      const dflash2_layer_weights& Ln = handle->layers[l + 1];
      conv_norm(nullptr, h1, parts, &P.down, int64_t(P.M) * H, Ln.conv_attn, Ln.dconv_attn,
                fp8 ? Ln.dconv_attn_scale : nullptr, Ln.attn_norm, h0);
    } else {
      norm(P.M, nullptr, bs, nullptr, h1, parts, &P.down, int64_t(P.M) * H, nullptr,
           handle->w.final_norm, debug_hidden, nbuf, 1);
    }
    if ((st = check_launch("draft_block/layer")) != DFLASH2_OK) return st;
  }

  // ---- 3. lm_head + top-k --------------------------------------------------
  LmHeadArgs la{};
  la.X = nbuf; la.ldx = H; la.W = handle->w.lm_head; la.ldw = H;
  la.scale = dt == DFLASH2_FP8_E4M3 ? handle->w.lm_head_scale : nullptr;
  la.M = P.Mh; la.N = c.vocab; la.K = H; la.M_dev = nullptr; la.groups = P.groups;
  la.k = c.selector_top_k; la.cand = reinterpret_cast<uint64_t*>(ws + P.off_cand);
  la.debug_logits = debug_logits;
  la.rs = normed;
  {
    const int64_t bytes = int64_t(c.vocab) * H * wb + (la.scale ? int64_t(c.vocab) * 4 : 0) +
                          int64_t(P.Mh) * H * ab + int64_t(P.Mh) * c.selector_top_k * 8 +
                          (debug_logits ? int64_t(P.Mh) * c.vocab * 4 : 0);
    traced(stream, DFLASH2_K_LMHEAD_TOPK, bytes, 2 * int64_t(P.Mh) * c.vocab * H,
           [&] { launch_lmhead_topk(dt, la, stream); });
  }
  TopkMergeArgs ma{};
  ma.cand = la.cand; ma.M = P.Mh; ma.k = c.selector_top_k;
  if (lmhead_tiled_ok(dt, P.Mh, H, c.selector_top_k)) {
    ma.glen = 16;
    ma.count = lmhead_tiled_lists(dt, P.Mh, c.vocab) * 16;
    ma.lstride = 16; ma.kstride = 1;
  } else {
    ma.glen = c.selector_top_k;
    ma.count = P.groups * c.selector_top_k;
    ma.lstride = 1; ma.kstride = P.groups;
  }
  ma.M_dev = nullptr; ma.ids = topk_ids; ma.vals = topk_vals;
  ma.multiplier = c.output_multiplier; ma.softcap = c.final_logit_softcapping;
  if (c.selector_top_k <= 16 && ma.count / ma.glen > 256) {
    // more than 256 lists per row (more than one per thread of the merge
    // kernel's block): fold them 64 at a time first, with one wave per 64
    // lists of a row (the weight-streaming lm_head writes one list per 128
    // ids: 1187 per row at a 151936 vocabulary; at batch 1, merge kernel +
    // selector 38.5 us per step, fold + merging selector 33.0)
    uint64_t* c2 = reinterpret_cast<uint64_t*>(ws + P.off_cand2);
    const int nc = topk_premerge_lists(ma.count / ma.glen);
    traced(stream, DFLASH2_K_TOPK_MERGE, int64_t(P.Mh) * ma.count * 8 + int64_t(P.Mh) * nc * 16 * 8, 0,
           [&] { launch_topk_premerge(ma, c2, stream); });
    ma.cand = c2; ma.count = nc * 16; ma.glen = 16; ma.lstride = 16; ma.kstride = 1;
  }
  if (path_idx && c.selector_top_k <= 16 && ma.count / ma.glen <= 64) {
    // ---- 4. candidate merge + path selector in one launch: the selector's
    // kernel merges the (at most 64) sorted lists of each row itself, one
    // wave per row and a block per sequence.  With 65-256 lists the merge
    // keeps its own kernel, a block per row (the tiled lm_head's 119-128
    // runs per row at the long-block and batched workloads: 39.3 / 32.2 us
    // per step against 45.6 / 33.7 folded and merged in the selector).
    SelectArgs a{};
    a.cand = ma.cand; a.count = ma.count; a.glen = ma.glen; a.lstride = ma.lstride; a.kstride = ma.kstride;
    a.anchors = anchor_ids; a.ids = topk_ids; a.vals = topk_vals;
    a.tl = handle->w.sel_tl; a.tr = handle->w.sel_tr;
    a.B = batch; a.P = c.block_size - 1; a.k = c.selector_top_k; a.r = c.selector_rank; a.V = c.vocab;
    a.path = path_idx; a.drafts = draft_tokens; a.score = path_score;
    a.multiplier = ma.multiplier; a.softcap = ma.softcap; a.ids_out = topk_ids; a.vals_out = topk_vals;
    const int64_t pairs = int64_t(batch) * (int64_t(a.P - 1) * a.k * a.k + a.k);
    const int64_t bytes = int64_t(P.Mh) * a.count * 8 + int64_t(P.Mh) * a.k * 8 +
                          int64_t(batch) * (a.P * a.k + 1) * 2 * a.r * 4 + int64_t(batch) * a.P * 8;
    traced(stream, DFLASH2_K_MERGE_SELECT, bytes, 2 * pairs * a.r,
           [&] { launch_select(a, select_window(a.k, a.r, a.P, kSelectLds), stream); });
    if ((st = check_launch("draft_select/lm_head")) != DFLASH2_OK) return st;
    return ok();
  }
  traced(stream, DFLASH2_K_TOPK_MERGE, int64_t(P.Mh) * ma.count * 8 + int64_t(P.Mh) * ma.k * 8, 0,
         [&] { launch_topk_merge(ma, stream); });
  if ((st = check_launch("draft_block/lm_head")) != DFLASH2_OK) return st;
  if (path_idx) return select_impl(handle, stream, batch, anchor_ids, topk_ids, topk_vals, path_idx, draft_tokens,
                                   path_score, nullptr, 0.0f, 0, 0, nullptr, nullptr, "draft_select");
  return ok();
}

dflash2_status dflash2_draft_block(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                   const int32_t* anchor_ids, const void* new_taps,
                                   const int32_t* new_offsets, const int32_t* ctx_lens,
                                   int64_t max_new_rows, void* k_cache, void* v_cache,
                                   int32_t* topk_ids, float* topk_vals, float* debug_logits,
                                   float* debug_hidden, void* workspace, size_t workspace_bytes) {
  return draft_impl(handle, stream, batch, anchor_ids, new_taps, new_offsets, ctx_lens, max_new_rows, k_cache,
                    v_cache, topk_ids, topk_vals, debug_logits, debug_hidden, workspace, workspace_bytes, nullptr,
                    nullptr, nullptr);
}

dflash2_status dflash2_draft_select(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                    const int32_t* anchor_ids, const void* new_taps,
                                    const int32_t* new_offsets, const int32_t* ctx_lens,
                                    int64_t max_new_rows, void* k_cache, void* v_cache, int32_t* topk_ids,
                                    float* topk_vals, int32_t* path_idx, int32_t* draft_tokens,
                                    float* path_score, float* debug_logits, void* workspace,
                                    size_t workspace_bytes) {
  if (!path_idx) return fail(DFLASH2_ERR_INVALID_ARG, "draft_select: null path_idx");
  const dflash2_status st = draft_impl(handle, stream, batch, anchor_ids, new_taps, new_offsets, ctx_lens,
                                       max_new_rows, k_cache, v_cache, topk_ids, topk_vals, debug_logits, nullptr,
                                       workspace, workspace_bytes, path_idx, draft_tokens, path_score);
  return st == DFLASH2_OK ? ok() : st;
}

}  // extern "C"

namespace {
dflash2_status select_impl(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                           const int32_t* anchor_ids, const int32_t* topk_ids, const float* topk_vals,
                           int32_t* path_idx, int32_t* draft_tokens, float* path_score, float* debug_pair,
                           float p_min, int32_t n_min, int32_t n_max, int32_t* draft_lens,
                           float* path_conf, const char* name) {
  if (!handle) return fail(DFLASH2_ERR_INVALID_ARG, "%s: null handle", name);
  const dflash2_config& c = handle->cfg;
  if (batch < 1 || batch > c.max_batch)
    return fail(DFLASH2_ERR_SHAPE, "%s: batch %d outside 1..max_batch %d", name, batch, c.max_batch);
  if (!anchor_ids || !topk_ids || !topk_vals || !path_idx || !draft_tokens)
    return fail(DFLASH2_ERR_INVALID_ARG, "%s: null pointer argument", name);
  if (!(p_min >= 0.0f && p_min <= 1.0f))
    return fail(DFLASH2_ERR_INVALID_ARG, "%s: p_min %g outside [0, 1]", name, double(p_min));
  SelectArgs a{};
  a.anchors = anchor_ids; a.ids = topk_ids; a.vals = topk_vals;
  a.tl = handle->w.sel_tl; a.tr = handle->w.sel_tr;
  a.B = batch; a.P = c.block_size - 1; a.k = c.selector_top_k; a.r = c.selector_rank; a.V = c.vocab;
  a.path = path_idx; a.drafts = draft_tokens; a.score = path_score; a.debug_pair = debug_pair;
  a.p_min = p_min; a.n_min = n_min; a.n_max = n_max; a.lens = draft_lens; a.conf = path_conf;
  {
    const bool stop = draft_lens || path_conf;
    const int64_t pairs = int64_t(batch) * (int64_t(a.P - 1) * a.k * a.k + a.k + (stop ? int64_t(a.P) * a.k : 0));
    const int64_t bytes = int64_t(batch) * a.P * a.k * 8 + int64_t(batch) * (a.P * a.k + 1) * 2 * a.r * 4 +
                          int64_t(batch) * a.P * 8 + (stop ? int64_t(batch) * (a.P + 1) * 4 : 0);
    traced(stream, DFLASH2_K_SELECT, bytes, 2 * pairs * a.r,
           [&] { launch_select(a, select_window(a.k, a.r, a.P, kSelectLds), stream); });
  }
  return check_launch(name);
}
}  // namespace

extern "C" {

dflash2_status dflash2_select_path(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                   const int32_t* anchor_ids, const int32_t* topk_ids,
                                   const float* topk_vals, int32_t* path_idx,
                                   int32_t* draft_tokens, float* path_score, float* debug_pair) {
  const dflash2_status st = select_impl(handle, stream, batch, anchor_ids, topk_ids, topk_vals, path_idx,
                                        draft_tokens, path_score, debug_pair, 0.0f, 0, 0, nullptr, nullptr,
                                        "select_path");
  return st == DFLASH2_OK ? ok() : st;
}

dflash2_status dflash2_select_path_stop(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                        const int32_t* anchor_ids, const int32_t* topk_ids,
                                        const float* topk_vals, float p_min, int32_t n_min,
                                        int32_t n_max, int32_t* path_idx, int32_t* draft_tokens,
                                        int32_t* draft_lens, float* path_conf, float* path_score) {
  if (!draft_lens) return fail(DFLASH2_ERR_INVALID_ARG, "select_path_stop: null draft_lens");
  const dflash2_status st = select_impl(handle, stream, batch, anchor_ids, topk_ids, topk_vals, path_idx,
                                        draft_tokens, path_score, nullptr, p_min, n_min, n_max, draft_lens,
                                        path_conf, "select_path_stop");
  return st == DFLASH2_OK ? ok() : st;
}

}  // extern "C"

namespace {
struct VerifyPlan {
  int nchunks, chunk;
  size_t bytes;
};
VerifyPlan plan_verify(int B, int bs, int V) {
  VerifyPlan v;
  const int64_t rows = int64_t(B) * bs;
  int64_t n = std::max<int64_t>(1, cdiv(2048, rows));
  n = std::min<int64_t>(n, std::max<int64_t>(1, cdiv(V, 4096)));
  v.chunk = int(cdiv(cdiv(V, n), 256) * 256);
  v.nchunks = int(cdiv(V, v.chunk));
  v.bytes = align_up(size_t(rows) * v.nchunks * 8);
  return v;
}
}  // namespace

extern "C" {

dflash2_status dflash2_verify_workspace_size(int32_t batch, int32_t block_size, int32_t vocab,
                                             size_t* bytes) {
  if (!bytes) return fail(DFLASH2_ERR_INVALID_ARG, "verify_workspace_size: null argument");
  if (!rows_ok(batch, block_size) || vocab < 1)
    return fail(DFLASH2_ERR_SHAPE, "verify_workspace_size: bad sizes");
  *bytes = plan_verify(batch, block_size, vocab).bytes;
  return ok();
}

}  // extern "C"

namespace {
dflash2_status greedy_impl(hipStream_t stream, int32_t batch, int32_t block_size, int32_t vocab,
                           const int32_t* draft_tokens, const int32_t* draft_lens, const float* target_logits,
                           int32_t* accepted, int32_t* bonus, int32_t* target_argmax, float* draft_prob,
                           void* workspace, const char* name) {
  const VerifyPlan vp = plan_verify(batch, block_size, vocab);
  VerifyArgs a{};
  a.drafts = draft_tokens; a.logits = target_logits;
  a.B = batch; a.bs = block_size; a.V = vocab; a.nchunks = vp.nchunks; a.chunk = vp.chunk;
  a.part = static_cast<uint64_t*>(workspace);
  a.accepted = accepted; a.bonus = bonus; a.argmax = target_argmax;
  a.lens = draft_lens; a.draft_prob = draft_prob;
  traced(stream, DFLASH2_K_VERIFY_PARTIAL, int64_t(batch) * block_size * vocab * 4, 0,
         [&] { launch_verify_partial(a, stream); });
  traced(stream, DFLASH2_K_VERIFY_FINAL, int64_t(batch) * (block_size - 1) * 4 + int64_t(batch) * 8, 0,
         [&] { launch_verify_final(a, stream); });
  return check_launch(name);
}

// Row results of the sampled verification: theta, max key, kept count
// [rows] u32; kept mass S, draft weight Ed [rows] u64; kept ids [rows][SV_OUT]
// u32 and weights [rows][SV_OUT] u64.
size_t sample_ws_bytes(int B, int bs) {
  const size_t rows = size_t(B) * bs;
  return align_up(rows * 4) * 3 + align_up(rows * 8) * 2 + align_up(rows * SV_OUT * 4) +
         align_up(rows * SV_OUT * 8);
}
}  // namespace

extern "C" {

dflash2_status dflash2_verify_accept(hipStream_t stream, int32_t batch, int32_t block_size,
                                     int32_t vocab, const int32_t* draft_tokens,
                                     const float* target_logits, int32_t* accepted,
                                     int32_t* bonus, int32_t* target_argmax, void* workspace,
                                     size_t workspace_bytes) {
  if (!rows_ok(batch, block_size) || vocab < 1)
    return fail(DFLASH2_ERR_SHAPE, "verify_accept: bad sizes (batch %d, block_size %d, vocab %d)",
                batch, block_size, vocab);
  if (!draft_tokens || !target_logits || !accepted || !bonus)
    return fail(DFLASH2_ERR_INVALID_ARG, "verify_accept: null pointer argument");
  const VerifyPlan vp = plan_verify(batch, block_size, vocab);
  if (!workspace || workspace_bytes < vp.bytes || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return fail(DFLASH2_ERR_WORKSPACE, "verify_accept: workspace needs %zu bytes, 256-aligned", vp.bytes);
  const dflash2_status st = greedy_impl(stream, batch, block_size, vocab, draft_tokens, nullptr, target_logits,
                                        accepted, bonus, target_argmax, nullptr, workspace, "verify_accept");
  return st == DFLASH2_OK ? ok() : st;
}

}  // extern "C"

// Scratch of dflash2_verify_accept_noalloc: the per-(row, vocabulary chunk)
// best keys of the greedy verifier, held in this library's own device array
// instead of a caller workspace.  Each GPU holds its own copy for the life
// of the process; every call on a GPU shares it, so calls that overlap on
// one GPU race.  The verifier overwrites every key it reads back, so
// nothing needs clearing between calls.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the stream's device, looked up once per
// device with that device current (the host-side name is not a device
// address).
dflash2_status scratch_address(hipStream_t stream, void** out, const char* name) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DFLASH2_ERR_HIP, "%s: device of the stream: %s", name, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH2_ERR_HIP, "%s: device %d out of range", name, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int prev = 0;
    if ((e = hipGetDevice(&prev)) != hipSuccess)
      return fail(DFLASH2_ERR_HIP, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
    if (prev != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(DFLASH2_ERR_HIP, "%s: hipSetDevice(%d): %s", name, dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != dev) (void)hipSetDevice(prev);
    if (e != hipSuccess || !p)
      return fail(DFLASH2_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", name, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DFLASH2_OK;
}
}  // namespace

extern "C" {

dflash2_status dflash2_verify_accept_noalloc(hipStream_t stream, int32_t batch, int32_t block_size,
                                             int32_t vocab, const int32_t* draft_tokens,
                                             const float* target_logits, int32_t* accepted,
                                             int32_t* bonus, int32_t* target_argmax) {
  if (!rows_ok(batch, block_size) || vocab < 1)
    return fail(DFLASH2_ERR_SHAPE, "verify_accept_noalloc: bad sizes (batch %d, block_size %d, vocab %d)",
                batch, block_size, vocab);
  if (!draft_tokens || !target_logits || !accepted || !bonus)
    return fail(DFLASH2_ERR_INVALID_ARG, "verify_accept_noalloc: null pointer argument");
  const VerifyPlan vp = plan_verify(batch, block_size, vocab);
  if (vp.bytes > kNoAllocScratchBytes)
    return fail(DFLASH2_ERR_WORKSPACE,
                "verify_accept_noalloc: needs %zu bytes of scratch, more than its built-in %zu "
                "(batch * block_size <= %zu); use dflash2_verify_accept with a workspace",
                vp.bytes, kNoAllocScratchBytes, kNoAllocScratchBytes / 8);
  void* ws = nullptr;
  dflash2_status st = scratch_address(stream, &ws, "verify_accept_noalloc");
  if (st != DFLASH2_OK) return st;
  st = greedy_impl(stream, batch, block_size, vocab, draft_tokens, nullptr, target_logits, accepted, bonus,
                   target_argmax, nullptr, ws, "verify_accept_noalloc");
  return st == DFLASH2_OK ? ok() : st;
}

dflash2_status dflash2_verify_sample_workspace_size(int32_t batch, int32_t block_size, int32_t vocab,
                                                    size_t* bytes) {
  if (!bytes) return fail(DFLASH2_ERR_INVALID_ARG, "verify_sample_workspace_size: null argument");
  if (!rows_ok(batch, block_size) || vocab < 1)
    return fail(DFLASH2_ERR_SHAPE, "verify_sample_workspace_size: bad sizes");
  *bytes = std::max(plan_verify(batch, block_size, vocab).bytes, sample_ws_bytes(batch, block_size));
  return ok();
}

dflash2_status dflash2_verify_sample(hipStream_t stream, int32_t batch, int32_t block_size, int32_t vocab,
                                     const int32_t* draft_tokens, const int32_t* draft_lens,
                                     const float* target_logits, const float* uniforms, float temperature,
                                     int32_t top_k, float top_p, int32_t* accepted, int32_t* bonus,
                                     float* draft_prob, void* workspace, size_t workspace_bytes) {
  if (!rows_ok(batch, block_size) || vocab < 1)
    return fail(DFLASH2_ERR_SHAPE, "verify_sample: bad sizes (batch %d, block_size %d, vocab %d)",
                batch, block_size, vocab);
  if (!draft_tokens || !target_logits || !accepted || !bonus)
    return fail(DFLASH2_ERR_INVALID_ARG, "verify_sample: null pointer argument");
  if (!(temperature >= 0.0f) || std::isinf(temperature))
    return fail(DFLASH2_ERR_INVALID_ARG, "verify_sample: temperature %g is not finite and >= 0",
                double(temperature));
  if (top_k < 0) return fail(DFLASH2_ERR_INVALID_ARG, "verify_sample: top_k %d < 0", top_k);
  if (!(top_p > 0.0f)) return fail(DFLASH2_ERR_INVALID_ARG, "verify_sample: top_p %g is not > 0", double(top_p));
  if (temperature > 0.0f && !uniforms)
    return fail(DFLASH2_ERR_INVALID_ARG, "verify_sample: null uniforms with temperature > 0");
  size_t need = 0;
  dflash2_verify_sample_workspace_size(batch, block_size, vocab, &need);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return fail(DFLASH2_ERR_WORKSPACE, "verify_sample: workspace needs %zu bytes, 256-aligned", need);
  dflash2_status st;
  if (temperature == 0.0f) {
    st = greedy_impl(stream, batch, block_size, vocab, draft_tokens, draft_lens, target_logits, accepted, bonus,
                     nullptr, draft_prob, workspace, "verify_sample");
  } else {
    int bits = 0;
    while ((int64_t(1) << bits) < int64_t(vocab)) ++bits;
    const size_t rows = size_t(batch) * block_size;
    char* ws = static_cast<char*>(workspace);
    SampleArgs a{};
    a.logits = target_logits; a.drafts = draft_tokens; a.lens = draft_lens; a.uni = uniforms;
    a.temp = temperature;
    a.top_k = (top_k >= vocab) ? 0 : top_k;
    a.top_p = top_p >= 1.0f ? 1.0f : top_p;
    a.qscale = std::ldexp(1.0f, 52 - bits);
    a.B = batch; a.bs = block_size; a.V = vocab;
    size_t off = 0;
    auto carve = [&](size_t bytes) { char* q = ws + off; off += align_up(bytes); return q; };
    a.theta = reinterpret_cast<uint32_t*>(carve(rows * 4));
    a.mkey = reinterpret_cast<uint32_t*>(carve(rows * 4));
    a.kept_n = reinterpret_cast<int32_t*>(carve(rows * 4));
    a.S = reinterpret_cast<uint64_t*>(carve(rows * 8));
    a.Ed = reinterpret_cast<uint64_t*>(carve(rows * 8));
    a.kept_id = reinterpret_cast<uint32_t*>(carve(rows * SV_OUT * 4));
    a.kept_w = reinterpret_cast<uint64_t*>(carve(rows * SV_OUT * 8));
    a.accepted = accepted; a.bonus = bonus; a.draft_prob = draft_prob;
    traced(stream, DFLASH2_K_SAMPLE_ROWS, int64_t(rows) * vocab * 4 + int64_t(rows) * 24, 0,
           [&] { launch_sample_rows(a, stream); });
    traced(stream, DFLASH2_K_SAMPLE_PICK, int64_t(batch) * vocab * 4 + int64_t(rows) * 28, 0,
           [&] { launch_sample_pick(a, stream); });
    st = check_launch("verify_sample");
  }
  return st == DFLASH2_OK ? ok() : st;
}

dflash2_status dflash2_draft_losses_workspace_size(int32_t batch, int32_t block_size, int32_t vocab,
                                                  size_t* bytes) {
  if (!bytes) return fail(DFLASH2_ERR_INVALID_ARG, "draft_losses_workspace_size: null argument");
  if (!rows_ok(batch, block_size) || vocab < 1)
    return fail(DFLASH2_ERR_SHAPE, "draft_losses_workspace_size: bad sizes");
  const VerifyPlan lp = plan_verify(batch, block_size - 1, vocab);
  *bytes = align_up(size_t(batch) * (block_size - 1) * lp.nchunks * 8) + align_up(size_t(batch) * 6 * 8);
  return ok();
}

dflash2_status dflash2_draft_losses(dflash2_handle* handle, hipStream_t stream, int32_t batch,
                                    const int32_t* anchor_ids, const int32_t* labels, const float* logits,
                                    const int32_t* topk_ids, const float* topk_vals, float loss_decay_gamma,
                                    float selector_loss_weight, float* block_ce, float* selector_ce,
                                    float* losses, void* workspace, size_t workspace_bytes) {
  if (!handle) return fail(DFLASH2_ERR_INVALID_ARG, "draft_losses: null handle");
  const dflash2_config& c = handle->cfg;
  if (batch < 1 || batch > c.max_batch)
    return fail(DFLASH2_ERR_SHAPE, "draft_losses: batch %d outside 1..max_batch %d", batch, c.max_batch);
  if (!anchor_ids || !labels || !logits || !topk_ids || !topk_vals || !losses)
    return fail(DFLASH2_ERR_INVALID_ARG, "draft_losses: null pointer argument");
  if (!(loss_decay_gamma > 0.0f))
    return fail(DFLASH2_ERR_INVALID_ARG, "draft_losses: loss_decay_gamma %g is not > 0", double(loss_decay_gamma));
  if (!std::isfinite(selector_loss_weight))
    return fail(DFLASH2_ERR_INVALID_ARG, "draft_losses: selector_loss_weight is not finite");
  size_t need = 0;
  dflash2_draft_losses_workspace_size(batch, c.block_size, c.vocab, &need);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return fail(DFLASH2_ERR_WORKSPACE, "draft_losses: workspace needs %zu bytes, 256-aligned", need);
  const int P = c.block_size - 1;
  const VerifyPlan lp = plan_verify(batch, P, c.vocab);
  LossArgs a{};
  a.logits = logits; a.labels = labels; a.anchors = anchor_ids; a.ids = topk_ids; a.vals = topk_vals;
  a.tl = handle->w.sel_tl; a.tr = handle->w.sel_tr;
  a.B = batch; a.P = P; a.V = c.vocab; a.k = c.selector_top_k; a.r = c.selector_rank;
  a.nchunks = lp.nchunks; a.chunk = lp.chunk;
  a.mult = c.output_multiplier; a.cap = c.final_logit_softcapping;
  a.gamma = loss_decay_gamma; a.sel_weight = selector_loss_weight;
  char* ws = static_cast<char*>(workspace);
  a.part = reinterpret_cast<float*>(ws);
  a.seq = reinterpret_cast<double*>(ws + align_up(size_t(batch) * P * lp.nchunks * 8));
  a.block_ce = block_ce; a.selector_ce = selector_ce; a.losses = losses;
  const int64_t rows = int64_t(batch) * P;
  traced(stream, DFLASH2_K_LOSS_ROWS, rows * c.vocab * 4, 0, [&] { launch_loss_rows(a, stream); });
  traced(stream, DFLASH2_K_LOSS_SEQ, rows * (8 + int64_t(a.k) * 8 + 8) + int64_t(batch) * 4 + 16,
         2 * rows * a.k * a.r, [&] { launch_loss_seq(a, stream); });
  const dflash2_status st = check_launch("draft_losses");
  return st == DFLASH2_OK ? ok() : st;
}

}  // extern "C"

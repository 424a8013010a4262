// Main loop shared by the compute-bound GEMMs (the LDS-tiled linears and the
// lm_head of many activation rows): a block tile of 256 weight rows x BM
// activation rows (BM = 256, 192 or 128), 4 waves in a 2 x 2 layout; wave
// (wv, wm) owns weight rows [128 wv, 128 wv + 128) of the tile against
// activation rows [BM/2 wm, BM/2 (wm + 1)): 4 x BM/64 tiles of
// v_mfma_f32_32x32x16_bf16 (up to 256 accumulators, one wave per SIMD).
// Both operands go from global memory straight into LDS (buffer loads to
// LDS: 16 bytes per lane, no register round trip; scalar base and stage
// offset, a fixed 32-bit offset per lane), 64 k per stage, with R = 2 or 3
// stage buffers (one or two stages of loads in flight); each stage buffer is
// its own LDS object, so the compiler waits only for the loads of the buffer
// it reads.  A stage's loads go out in parts spread over the MFMAs.  Rows are 128 bytes
// (activations, bf16 weights) or 64 bytes (fp8 weights) with the 16-byte
// chunks of row r XOR-permuted by (r ^ (r >> 2)): the 32 x 32 x 16 operand
// reads (row = lane % 32, chunk by lane / 32) then hit distinct banks
// (measured on MI355X: one LDS cycle per 256 bytes, where an unpermuted
// layout takes eight and a (r + r / 8) permutation two).  fp8 weights read
// 16 bytes per lane for two k steps (the k order inside each pair of steps is
// permuted on both operands alike) and are widened to bf16 (exact) before
// the MFMA.  Within a stage, the operand reads of step s + 1 are interleaved
// with the MFMAs of step s; the barrier that hands over the next stage sits
// before the last step's MFMAs, which then overlap the first reads of the
// next stage and the loads of the stage after.
#pragma once

#include "common.h"

namespace dfl {

constexpr int kDmaBN = 256;  // weight rows per tile
constexpr int kDmaKT = 64;   // contraction depth per stage

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 16 bytes per lane from global memory straight into LDS at l + 16 * lane
// (l wave-uniform).  A non-template wrapper keeps the device-only builtin out
// of the host pass's instantiation of the kernel templates.
__device__ __forceinline__ void lds_load16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}

// The same through a buffer resource: 16 bytes per lane at byte offset
// voff + soff of the resource's base (soff wave-uniform).
__device__ __forceinline__ void lds_load16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* l) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)l, 16, voff, soff, 0, 0);
}

// raw buffer resource over [base, base + 4 GiB) (gfx9 data-format word)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(0xFFFFFFFFu), 0x00020000);
}

// A wave-uniform value kept in scalar registers (the caller guarantees that
// every lane holds the same value; the compiler cannot always prove it, and
// a buffer resource or scalar offset it takes for divergent is loaded in a
// loop over the lanes' distinct values).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

// 16-byte chunk permutation of an LDS row
__device__ __forceinline__ int chunk_perm(int r) { return r ^ (r >> 2); }

// s_waitcnt immediate: at most vm vector-memory operations outstanding, no
// LDS/scalar operation outstanding, export count untouched (gfx9 layout:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

template <typename TW, int BM, int R = 2, int NP = (R == 3 ? 4 : 2)>
struct DmaTile {
  static_assert(R == 2 || R == 3, "two or three stage buffers");
  static constexpr int SW = int(sizeof(TW));
  static constexpr int WROW = kDmaKT * SW, XROW = kDmaKT * 2;   // LDS bytes per row and stage
  static constexpr int WBYTES = kDmaBN * WROW, XBYTES = BM * XROW;
  static constexpr int WM = BM / 2, FJ = WM / 32;
  static constexpr int WLD = WBYTES / 4096, XLD = XBYTES / 4096;  // loads per wave and stage
  static constexpr int WCH = WROW / 16;                        // 16-byte chunks per weight row

  // Tile row t (0..255) holds weight row wrow(t) = nw_w + t - 64 w, where
  // w = t / 64 and nw_w is the nw argument of wave w (each wave loads tile
  // rows [64 w, 64 w + 64); nw = n0 + 64 w gives 256 consecutive rows).
  // acc[i][j][4 q + e] = sum over k in [kb, kb + 64 nk) of
  // W[wrow(128 wv + 32 i + 8 q + 4 h + e)][k] * X[m0 + WM wm + 32 j + r][k]
  // for lane (r, h) = (lane % 32, lane / 32) of wave (wv, wm).  Rows past
  // N / Mact are clamped to the last row (their results are never used).
  // wave and nw must be wave-uniform.
  __device__ __forceinline__ static void run(const bf16_t* __restrict__ X, int64_t ldx, const TW* __restrict__ W,
                                             int64_t ldw, int N, int Mact, int nw, int m0, int kb, int nk,
                                             int wave, char* w0, char* w1, char* w2, char* x0, char* x1, char* x2,
                                             f32x16 (&acc)[4][FJ]) {
    // An empty asm makes the lane index opaque, so the per-lane offsets below
    // are recomputed on every call rather than hoisted out of the caller's
    // tile loop and kept (spilled) across its epilogue.
    int lane = threadIdx.x & (WAVE - 1);
    asm volatile("" : "+v"(lane));
    const int wv = wave & 1, wm = wave >> 1;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) acc[i][j] = f32x16{};
    // 64-bit bases (the wave's first weight row, the block's first activation
    // row, at k = kb); per-lane 32-bit offsets below them (at most 64 weight
    // rows and 256 activation rows of at most 2^20 elements)
    const int wb0 = min(nw, N - 1), xb0 = min(m0, Mact - 1);
    const char* wbase = reinterpret_cast<const char*>(W) + (int64_t(wb0) * ldw + kb) * SW;
    const char* xbase = reinterpret_cast<const char*>(X) + (int64_t(xb0) * ldx + kb) * 2;
    uint32_t woff[WLD], xoff[XLD];
#pragma unroll
    for (int q = 0; q < WLD; ++q) {
      const int piece = wave * WLD + q;                   // 1 KB piece of the stage
      const int rpp = 1024 / WROW;                        // rows per piece
      const int row = rpp * piece + lane / WCH;           // tile row, in [64 wave, 64 wave + 64)
      const int chunk = (lane % WCH) ^ (chunk_perm(row) & (WCH - 1));
      woff[q] = uint32_t(min(nw + row - 64 * wave, N - 1) - wb0) * uint32_t(ldw) * SW + 16u * chunk;
    }
#pragma unroll
    for (int q = 0; q < XLD; ++q) {
      const int piece = wave * XLD + q;
      const int row = 8 * piece + (lane >> 3);
      const int chunk = (lane & 7) ^ (chunk_perm(row) & 7);
      xoff[q] = uint32_t(min(m0 + row, Mact - 1) - xb0) * uint32_t(ldx) * 2 + 16u * chunk;
    }
    // load q of a stage (weights first, then activations); a stage's loads
    // go out in NPART parts of PQ
    constexpr int NL = WLD + XLD, NPART = NP, PQ = (NL + NPART - 1) / NPART;
    static_assert(NPART >= 1 && NPART <= 4, "a stage's loads go out in one to four parts");
    // Buffer loads: the wave-uniform stage offset goes in a scalar register
    // and each lane's offset stays fixed, so a load needs no address
    // arithmetic on the lanes.
    const __amdgpu_buffer_rsrc_t wrs = raw_rsrc(uniform_ptr(wbase)), xrs = raw_rsrc(uniform_ptr(xbase));
    auto load_part = [&](int kt, char* wd, char* xd, int part) {
#pragma unroll
      for (int q = part * PQ; q < (part + 1) * PQ && q < NL; ++q) {
        const uint32_t kts = __builtin_amdgcn_readfirstlane(kt);
        if (q < WLD) lds_load16_buf(wrs, woff[q], kts * WROW, wd + 1024 * (wave * WLD + q));
        else lds_load16_buf(xrs, xoff[q - WLD], kts * XROW, xd + 1024 * (wave * XLD + q - WLD));
      }
    };
    auto load_stage = [&](int kt, char* wd, char* xd) {
#pragma unroll
      for (int part = 0; part < NPART; ++part) load_part(kt, wd, xd, part);
    };
    // operand read offsets: weights per (i, step) (bf16) or (i, pair of
    // steps) (fp8); activations per (j, step)
    int wrd[4][4], xrd[FJ][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 128 * wv + 32 * i + r;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int c = SW == 2 ? 2 * s + h : 2 * (s >> 1) + h;
        wrd[i][s] = row * WROW + 16 * (c ^ (chunk_perm(row) & (WCH - 1)));
      }
    }
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int row = WM * wm + 32 * j + r;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // fp8: step s, half h covers k = 32 (s / 2) + 16 h + 8 (s % 2) + 0..7
        const int c = SW == 2 ? 2 * s + h : 4 * (s >> 1) + 2 * h + (s & 1);
        xrd[j][s] = row * XROW + 16 * (c ^ (chunk_perm(row) & 7));
      }
    }
    u32x4 wr[2][4];     // bf16: by step parity; fp8: raw bytes of a pair of steps, by pair parity
    bf16x8 xr[2][FJ];   // by step parity
    auto prefetch = [&](int s, const char* wl, const char* xl) {
      if (SW == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[s & 1][i] = *reinterpret_cast<const u32x4*>(wl + wrd[i][s]);
      } else if ((s & 1) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) wr[(s >> 1) & 1][i] = *reinterpret_cast<const u32x4*>(wl + wrd[i][s]);
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) xr[s & 1][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xl + xrd[j][s]));
    };
    auto mfmas = [&](int s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Frag8Bf16 a;
        if (SW == 2) {
          a.v = __builtin_bit_cast(bf16x8, wr[s & 1][i]);
        } else {
          const u32x4 w = wr[(s >> 1) & 1][i];
          fp8x8_to_frag(a, (s & 1) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]});
        }
#pragma unroll
        for (int j = 0; j < FJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, xr[s & 1][j], acc[i][j], 0, 0, 0);
      }
    };
    auto nreads = [&](int s) { return FJ + ((SW == 2 || (s & 1) == 0) ? 4 : 0); };
    // one MFMA, then one DS read (while reads remain), ...; the nvm global
    // loads spread evenly over the step's MFMAs
    auto interleave = [&](int nrd, int nvm) {
      const int gap = nvm > 0 ? (4 * FJ) / nvm : 1;
#pragma unroll
      for (int q = 0; q < 4 * FJ; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (nvm > 0 && q % gap == 0 && q / gap < nvm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        if (q < nrd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    auto part_size = [&](int part) { return (part + 1) * PQ <= NL ? PQ : (part * PQ < NL ? NL - part * PQ : 0); };
    // One stage on (wl, xl), whose step 0 operands are already requested;
    // the next stage is in (wn, xn); after the barrier the loads of stage
    // kt_load go into (wl, xl), which no wave reads any more.  Before the
    // barrier each wave waits for its loads of the next stage (with three
    // buffers the loads of the stage after it stay in flight) and for its
    // reads of this one.  A stage's loads go out in NP parts: the first
    // after the barrier, the others (of the previous stage's kt_load, into
    // (wp, xp)) in steps 0-2 of the next stage, so that the MFMAs do not
    // wait behind the issue of a burst of loads.  Measured on the fp8
    // high-batch lm_head (1792 x 151936 x 5120): its main loop took 1.30x
    // the time of the same loop with the global loads switched off when each
    // wave issued its 12 loads per stage in one burst, 1.19x in four parts.
    // With two buffers the later parts land before that next stage's
    // barrier.
    auto stage = [&](char* wl, char* xl, const char* wn, const char* xn, int kt_load, char* wp, char* xp,
                     int kt_prev) {
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        if constexpr (NPART > 1) load_part(kt_prev, wp, xp, s + 1);
        prefetch(s + 1, wl, xl);
        mfmas(s);
        interleave(nreads(s + 1), NPART > 1 ? part_size(s + 1) : 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (R == 2) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      } else {
        // a workgroup fence would wait for every load in flight; the wait
        // above covers what the barrier must order (LDS only)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(WLD + XLD));
        asm volatile("s_barrier" ::: "memory");
      }
      __builtin_amdgcn_sched_barrier(0);
      load_part(kt_load, wl, xl, 0);
      prefetch(0, wn, xn);
      mfmas(3);
      interleave(nreads(0), part_size(0));
      __builtin_amdgcn_sched_barrier(0);
    };
    // Loads past the last stage repeat the last stage, so every stage has
    // the same loads in flight and the wait counts stay exact.
    int kt = 0;
    if constexpr (R == 2) {
      load_stage(0, w0, x0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // stage 1: the first part here, the others in stage 0
      load_part(min(1, nk - 1), w1, x1, 0);
      prefetch(0, w0, x0);
      int kp = min(1, nk - 1);
      for (; kt + 2 <= nk; kt += 2) {
        stage(w0, x0, w1, x1, min(kt + 2, nk - 1), w1, x1, kp);
        stage(w1, x1, w0, x0, min(kt + 3, nk - 1), w0, x0, min(kt + 2, nk - 1));
        kp = min(kt + 3, nk - 1);
      }
      if (kt < nk) stage(w0, x0, w1, x1, nk - 1, w1, x1, kp);
    } else {
      load_stage(0, w0, x0);
      load_stage(min(1, nk - 1), w1, x1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(WLD + XLD));
      asm volatile("s_barrier" ::: "memory");
      // stage 2: the first part here, the others in stage 0
      load_part(min(2, nk - 1), w2, x2, 0);
      prefetch(0, w0, x0);
      int kp = min(2, nk - 1);
      for (; kt + 3 <= nk; kt += 3) {
        stage(w0, x0, w1, x1, min(kt + 3, nk - 1), w2, x2, kp);
        stage(w1, x1, w2, x2, min(kt + 4, nk - 1), w0, x0, min(kt + 3, nk - 1));
        stage(w2, x2, w0, x0, min(kt + 5, nk - 1), w1, x1, min(kt + 4, nk - 1));
        kp = min(kt + 5, nk - 1);
      }
      if (kt < nk) stage(w0, x0, w1, x1, nk - 1, w2, x2, kp);
      if (kt + 1 < nk) stage(w1, x1, w2, x2, nk - 1, w0, x0, nk - 1);
    }
    __builtin_amdgcn_s_waitcnt(0);   // the last (repeated) loads have landed before LDS is reused
  }
};

}  // namespace dfl

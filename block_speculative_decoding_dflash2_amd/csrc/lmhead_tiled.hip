// lm_head + top-k for many activation rows (the batched and fp8 high-batch
// workloads), where every lm_head row meets hundreds of activation rows and
// the matrix cores set the pace.
//
// Main loop: the DMA tile of dma_tile.h (256 vocabulary rows x BM = 256 or
// 128 activation rows per block, both operands loaded straight into LDS),
// with three stage buffers where they fit in LDS.
//
// Measured at the fp8 high-batch shape (1792 x 151936 x 5120, random data):
// the main loop alone 2.27 ms (1.23 PF/s); with the global loads switched off
// 1.83 ms, which is the matrix-core rate this chip sustains on random
// operands (the same loop on all-zero operands runs at 82-86% of the nominal
// peak, on random ones at 61%); the loads alone 1.25 ms.
//
// Top-k.  A block sweeps a run of consecutive 256-id vocabulary tiles for
// its activation rows and keeps each row's 16 best keys (value desc, id asc)
// of the run in the row's output list cand[m][run][0..16), which the merge
// kernel reduces to the final k.  Per tile, each lane holds 64 logits of each
// of its rows; it inserts those that beat the row's current 16th key into a
// sorted list of 16 (after the first tile of a run few values qualify); the
// lists of the two half-waves holding a row merge by shuffle, those of the
// two waves through LDS, and the result merges with the run's list so far.
// Every step is an exact ranking, so ties and -0.0 follow the key order.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "dma_tile.h"
#include "kernels.h"

namespace dfl {

namespace {
constexpr int kLBN = kDmaBN;  // vocabulary rows per tile
constexpr int kLKT = kDmaKT;  // contraction depth per stage
}  // namespace

struct LmTiledArgs {
  const bf16_t* X; int64_t ldx;   // [M][K]
  const void* W; int64_t ldw;     // [V][K]
  const float* scale;             // [V] or null
  int M, N, K;
  const int32_t* M_dev;
  RowScale rs;
  uint64_t* cand;                 // [M][runs][16]
  float* debug_logits;            // [M][N] or null
  int nM, runs, tpb, nN;
};


// L (16 keys, largest first) <- the 16 largest of L and x.
__device__ __forceinline__ void insert_key(uint64_t (&L)[16], uint64_t x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool c = x > L[i];
    const uint64_t t = L[i];
    L[i] = c ? x : t;
    x = c ? t : x;
  }
}

// a (16 keys) sorted descending in place (bitonic network).
__device__ __forceinline__ void sort16_keys_desc(uint64_t (&a)[16]) {
#pragma unroll
  for (int size = 2; size <= 16; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ stride;
        if (l > i) {
          const bool desc = (i & size) == 0;
          const uint64_t x = a[i], y = a[l];
          const bool sw = desc ? (y > x) : (x > y);
          a[i] = sw ? y : x;
          a[l] = sw ? x : y;
        }
      }
}

// a (16 floats) sorted descending in place.
__device__ __forceinline__ void sort16_desc(float (&a)[16]) {
#pragma unroll
  for (int size = 2; size <= 16; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ stride;
        if (l > i) {
          const bool desc = (i & size) == 0;
          const float hi = fmaxf(a[i], a[l]), lo = fminf(a[i], a[l]);
          a[i] = desc ? hi : lo;
          a[l] = desc ? lo : hi;
        }
      }
}

// Per tile and row, only values that can still enter the row's 16 best are
// looked at:
//  * first tile of a run: each lane keeps the largest and second largest of
//    each group of 16 of its values; the 16th largest of a row's 32 such
//    values is a bound T with at least 16 of the row's values >= T, so no
//    value below T can be among the row's best 16;
//  * later tiles: the row's current 16th key.
// Passing values (about 18 of a row's 256 on a first tile, rarely any later)
// are staged in LDS by the lanes of rows that have some and inserted into
// the lane's sorted list of 16; rows whose lanes found nothing keep their
// list untouched.
template <typename TW, int BM, int R>
__global__ __launch_bounds__(256) void lmhead_tiled_kernel(LmTiledArgs p) {
  typedef DmaTile<TW, BM, R> T;
  constexpr int FJ = T::FJ, WM = T::WM;
  __shared__ __attribute__((aligned(1024))) char w0[T::WBYTES];
  __shared__ __attribute__((aligned(1024))) char w1[T::WBYTES];
  __shared__ __attribute__((aligned(1024))) char w2[R == 3 ? T::WBYTES : 16];
  __shared__ __attribute__((aligned(1024))) char x0[T::XBYTES];
  __shared__ __attribute__((aligned(1024))) char x1[T::XBYTES];
  __shared__ __attribute__((aligned(1024))) char x2[R == 3 ? T::XBYTES : 16];
  __shared__ float inv[BM];
  __shared__ float thr[BM];       // first tile of a run: the bound T
  __shared__ uint64_t thrk[BM];   // the row's current 16th key of the run (0: fewer than 16 so far)
  __shared__ f32x4 vscale4[kLBN / 4];  // the tile's per-vocabulary-row scales (1 without them)
  __shared__ int cnt[BM];         // keys appended to the row's slots in this tile
  // block -> (row tile, run of vocabulary tiles); blocks of one run are adjacent
  const int per = gridDim.x >> 3;
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= p.nM * p.runs) return;
  const int mt = t % p.nM, rg = t / p.nM;
  const int nt0 = rg * p.tpb, nt1 = min(p.nN, nt0 + p.tpb);
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m0 = mt * BM;
  if (m0 >= Mact || nt0 >= nt1) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 1, wm = wave >> 1;
  const int r = lane & 31, h = lane >> 5;
  for (int q = tid; q < BM; q += blockDim.x) {
    float v = 1.f;
    const int m = m0 + q;
    if (p.rs.sumsq && m < Mact) {
      const float s = sum_in_order(p.rs.sumsq + int64_t(m) * p.rs.blocks, p.rs.blocks);
      v = 1.0f / sqrtf(s * p.rs.inv_width + p.rs.eps);
    }
    inv[q] = v;
    thrk[q] = 0ull;
    cnt[q] = 0;
  }
  // (inv and thrk are read after the main loop's barriers)
  const TW* W = static_cast<const TW*>(p.W);
  const int nk = p.K / kLKT;
  for (int nt = nt0; nt < nt1; ++nt) {
    const int n0 = nt * kLBN;
    const bool fresh = nt == nt0;
    // (the previous tile's epilogue ended with a barrier; vscale is read
    // after the main loop's barriers)
    if (tid < kLBN / 4) {
      f32x4 sv = {1.f, 1.f, 1.f, 1.f};
      const int n = n0 + 4 * tid;
      if (sizeof(TW) == 1 && p.scale) {
        if (n + 3 < p.N) {
          sv = *reinterpret_cast<const f32x4*>(p.scale + n);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[e] = p.scale[min(n + e, p.N - 1)];
        }
      }
      vscale4[tid] = sv;
    }
    f32x16 acc[4][FJ];
    T::run(p.X, p.ldx, W, p.ldw, p.N, Mact, n0 + 64 * wave, m0, 0, nk, wave, w0, w1, w2, x0, x1, x2, acc);
    // lane (r, h) of wave (wv, wm): value 4 q + e of acc[i][j] is vocabulary id
    // n0 + lb + 32 i + 8 q + e, lb = 128 wv + 4 h, of local row WM wm + 32 j + r.
    // Per-lane values are recomputed per tile (see DmaTile::run).
    auto voff = [](int k) { return 32 * (k >> 4) + 8 * ((k & 15) >> 2) + (k & 3); };
    int lb = 128 * wv + 4 * h;
    asm volatile("" : "+v"(lb));
    const int nvalid = p.N - n0 - lb;   // ids at offsets < nvalid exist
    // bit k of vmask[hf]: the id of value k of half hf exists (all bits set
    // but in a ragged last tile)
    const bool ragged = n0 + kLBN > p.N;
    uint32_t vmask[2] = {~0u, ~0u};
    if (ragged) {
      vmask[0] = vmask[1] = 0u;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        vmask[0] |= uint32_t(voff(k) < nvalid) << k;
        vmask[1] |= uint32_t(64 + voff(k) < nvalid) << k;
      }
    }
    __syncthreads();  // every wave's loads have landed and the stage buffers are free
    // The run's list so far of row tid goes straight into LDS now (no
    // registers held across the appends below) and is read by the same lane
    // in the merge: 128 bytes per row, chunk q of the row of lane l of wave
    // w at glist + 8192 w + 1024 q + 16 l, in the upper halves of the bf16
    // weight stage buffers or the third activation stage buffer (fp8).
    static_assert(sizeof(TW) == 2 ? T::WBYTES >= 32768 : (R == 3 && T::XBYTES >= BM * 128),
                  "the lists fit beside the staging area");
    char* glist = sizeof(TW) == 2 ? (wave < 2 ? w0 : w1) + 16384 + (wave & 1) * 8192 : x2 + wave * 8192;
    if (!fresh && 64 * wave < BM) {
      const uint64_t* o = p.cand + (int64_t(min(m0 + tid, p.M - 1)) * p.runs + rg) * 16;
#pragma unroll
      for (int q = 0; q < 8; ++q) lds_load16(o + 2 * q, glist + 1024 * q);
    }

    // Logits of the lane's 32 values of row j, half hf (vocabulary offsets
    // lb + 64 hf + voff(k), k < 32), copied out of the accumulators by a
    // switch on (j, hf), so that a single copy of the code below, in loops
    // that are not unrolled, serves every row: unrolled per row it would not
    // fit the instruction cache.
    // (sv: the per-vocabulary-row scales of half hf, fp8 weights only)
    auto load_sv = [&](int hf, float (&sv)[32]) {
      if constexpr (sizeof(TW) == 1) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          const f32x4 v4 = vscale4[(lb + 64 * hf + voff(4 * g)) >> 2];
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[4 * g + e] = v4[e];
        }
      }
    };
    auto logits_half_sv = [&](int jh, float (&x)[32], const float (&sv)[32]) {
      // (an empty asm over the accumulators stops the compiler from hoisting
      // their copies out of the loops that call this, which ran the 192-row
      // kernel out of registers)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < FJ; ++jj) asm volatile("" : "+a"(acc[i][jj]));
      const int j = jh >> 1;
      const float iv = inv[WM * wm + 32 * j + r];
      auto take = [&](auto J, auto HF) {
        constexpr int jj = decltype(J)::value, hh = decltype(HF)::value;
        if constexpr (jj < FJ) {
#pragma unroll
          for (int k = 0; k < 32; ++k) x[k] = acc[2 * hh + (k >> 4)][jj][k & 15];
        }
      };
      if (jh >= 2 * FJ) __builtin_unreachable();
      switch (jh) {
        case 0: take(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}); break;
        case 1: take(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}); break;
        case 2: take(std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}); break;
        case 3: take(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}); break;
        case 4: take(std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{}); break;
        case 5: take(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}); break;
        case 6: take(std::integral_constant<int, 3>{}, std::integral_constant<int, 0>{}); break;
        default: take(std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{}); break;
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        float y = x[k];
        if constexpr (sizeof(TW) == 1) y *= sv[k];   // (bf16 weights have no scales)
        x[k] = y * iv;   // (-0.0 is ranked as +0.0 by the key)
      }
    };
    auto logits_half = [&](int jh, float (&x)[32]) {
      float sv[32];
      load_sv(jh & 1, sv);
      logits_half_sv(jh, x, sv);
    };
    static_assert(FJ <= 4, "at most four row blocks per wave");
    // bit k: value x[k] can enter the row's list (ids past the vocabulary
    // never do).  Branch-free: first tile of a run, x >= T; later, the key
    // beats the row's 16th key tk (any number while the list is not full).
    auto pass_mask = [&](const float (&x)[32], int base, int hf, float tf, float tv, uint32_t tlo, bool tk0) {
      uint32_t mask = 0u;
      if (fresh) {
#pragma unroll
        for (int k = 0; k < 32; ++k)
          mask |= (uint32_t(x[k] >= tf) & uint32_t(64 * hf + voff(k) < nvalid)) << k;
      } else {
        const uint32_t any = uint32_t(tk0);
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const float y = x[k];
          const uint32_t beats = uint32_t(y > tv) |
                                 (uint32_t(y == tv) & uint32_t(0xFFFFFFFFu - uint32_t(n0 + base + voff(k)) > tlo));
          const uint32_t ok = (any & uint32_t(y == y)) | beats;
          mask |= (ok & uint32_t(64 * hf + voff(k) < nvalid)) << k;
        }
      }
      return mask;
    };

    // 1. first tile of a run: the bound T of each row
    if (fresh) {
      float* ab = reinterpret_cast<float*>(x0);  // [32 slots][BM rows]
#pragma nounroll
      for (int jh = 0; jh < 2 * FJ; ++jh) {
        float x[32];
        logits_half(jh, x);
        const int lm = WM * wm + 32 * (jh >> 1) + r;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          float a = -INFINITY, b = -INFINITY;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const float y = (vmask[jh & 1] >> (16 * ii + v)) & 1u ? x[16 * ii + v] : -INFINITY;
            b = fmaxf(b, fminf(a, y));
            a = fmaxf(a, y);
          }
          const int slot = ((wv * 2 + h) * 4 + 2 * (jh & 1) + ii) * 2;
          ab[slot * BM + lm] = a;
          ab[(slot + 1) * BM + lm] = b;
        }
      }
      __syncthreads();
      if (tid < BM) {
        // the 16 largest of the union of the sorted maxima A and second
        // maxima B are max(A[q], B[15 - q]); T is their minimum
        float A[16], B[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          A[q] = ab[(2 * q) * BM + tid];
          B[q] = ab[(2 * q + 1) * BM + tid];
        }
        sort16_desc(A);
        sort16_desc(B);
        float Tb = INFINITY;
#pragma unroll
        for (int q = 0; q < 16; ++q) Tb = fminf(Tb, fmaxf(A[q], B[15 - q]));
        thr[tid] = Tb;
      }
      __syncthreads();
    }

    // 2. common path.  The debug copy first (only when asked for); then every
    // lane compares each of its values with the row's bound (first tile: T;
    // later: the value of the row's 16th key, ties passing, since the id
    // order is settled by the exact key comparison of the insertion below;
    // any value while the list is not full) and appends the keys of those
    // that pass to the row's slots in LDS (one atomic per lane and row).
    // Slots of rows [0, WM) are in x0, of rows [WM, BM) in x1 (free now: the
    // bounds above were read before the last barrier).
    constexpr int NSLOT = 32;
    static_assert(WM * NSLOT * 8 <= T::XBYTES, "slots fit an activation stage buffer");
    float* stg = reinterpret_cast<float*>(wave < 2 ? w0 : w1) + (wave & 1) * 32 * WAVE;  // [32][64] per wave
    static_assert(2 * 32 * WAVE * 4 <= T::WBYTES, "staging fits a weight stage buffer");
    // Slot q of row lm sits at position q ^ (lm % 32) of the row's 32: rows
    // are 256 bytes apart, so without the swizzle the 32 rows of a wave's
    // lanes would all hit the same LDS banks.
    auto slots_of = [&](int lm) {
      return reinterpret_cast<uint64_t*>(lm < WM ? x0 : x1) + (lm % WM) * NSLOT;
    };
    if (p.debug_logits) {
#pragma nounroll
      for (int jh = 0; jh < 2 * FJ; ++jh) {
        float x[32];
        logits_half(jh, x);
        const int m = m0 + WM * wm + 32 * (jh >> 1) + r;
        const int hf = jh & 1;
        if (m < Mact) {
          float* row = p.debug_logits + int64_t(m) * p.N + n0 + lb + 64 * hf;
#pragma unroll
          for (int g = 0; g < 8; ++g) {
            const int off = voff(4 * g);
            float* dst = row + off;
            if (64 * hf + off + 3 < nvalid && (p.N & 3) == 0) {
              *reinterpret_cast<f32x4*>(dst) = f32x4{x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (64 * hf + off + e < nvalid) dst[e] = x[4 * g + e];
            }
          }
        }
      }
    }
    // (fp8: half-major, so that a half's scales are read once; the bounds of
    // the lane's rows are read before the loop, so no LDS wait heads it)
    float tes[FJ];
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int lm = WM * wm + 32 * j + r;
      const uint64_t tk = thrk[lm];
      tes[j] = fresh ? thr[lm] : (tk == 0ull ? -__FLT_MAX__ : key_val(tk));
    }
    float sv[32];
#pragma nounroll
    for (int it = 0; it < 2 * FJ; ++it) {
      const int j = sizeof(TW) == 1 ? it % FJ : it >> 1, hf = sizeof(TW) == 1 ? it / FJ : it & 1;
      if (j == 0) load_sv(hf, sv);
      const int jh = 2 * j + hf;
      const int lm = WM * wm + 32 * j + r;
      const int base = lb + 64 * hf;   // vocabulary offset of x[0] in the tile
      float te = tes[0];
#pragma unroll
      for (int q = 1; q < FJ; ++q) te = j == q ? tes[q] : te;
      float x[32];
      logits_half_sv(jh, x, sv);
      uint32_t mk = 0u;
#pragma unroll
      for (int k = 0; k < 32; ++k) mk |= uint32_t(x[k] >= te) << k;
      mk &= vmask[jh & 1];
      if (mk != 0u) {
        // stage the 32 values (lane-major, wave-private) and visit the set
        // bits, four per round, so that their LDS reads overlap
#pragma unroll
        for (int k = 0; k < 32; ++k) stg[k * WAVE + lane] = x[k];
        uint64_t* sl = slots_of(lm);
        int pos = atomicAdd(&cnt[lm], __builtin_popcount(mk));
        while (mk != 0u) {
          int kk[4];
          uint32_t live = 0u;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            kk[u] = mk != 0u ? __builtin_ctz(mk) : 0;
            live |= uint32_t(mk != 0u) << u;
            mk &= mk - 1u;
          }
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = stg[kk[u] * WAVE + lane];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (((live >> u) & 1u) && pos < NSLOT) sl[pos ^ r] = rank_key(v[u], uint32_t(n0 + base + voff(kk[u])));
            pos += int((live >> u) & 1u);
          }
        }
      }
    }
    if (!__syncthreads_or(tid < BM && cnt[tid] > NSLOT)) {
      if (tid < BM) {
        const int lm = tid, m = m0 + lm;
        const int c = cnt[lm];
        if (m < Mact && (c > 0 || fresh)) {
          uint64_t* o = p.cand + (int64_t(m) * p.runs + rg) * 16;
          // the new keys, 16 at a time: sorted, then merged with the list
          // (a sorting network and a half-cleaner cascade: short dependency
          // chains, unlike one insertion per key)
          const uint64_t* sl = slots_of(lm);
          uint64_t G[16];
          if (fresh) {
#pragma unroll
            for (int q = 0; q < 16; ++q) G[q] = 0ull;
          } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // this lane's list has landed in LDS
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const u32x4 v = *reinterpret_cast<const u32x4*>(glist + 1024 * q + 16 * lane);
              G[2 * q] = uint64_t(v[0]) | (uint64_t(v[1]) << 32);
              G[2 * q + 1] = uint64_t(v[2]) | (uint64_t(v[3]) << 32);
            }
          }
          for (int q0 = 0; q0 < c; q0 += 16) {
            uint64_t Nk[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) Nk[q] = q0 + q < c ? sl[(q0 + q) ^ (lm & 31)] : 0ull;
            sort16_keys_desc(Nk);
            uint64_t rev[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) rev[q] = Nk[15 - q];
            bitonic_top<16>(G, rev);
          }
#pragma unroll
          for (int q = 0; q < 16; ++q) o[q] = G[q];
          thrk[lm] = G[15];
        } else if (m >= Mact) {
          thrk[lm] = ~0ull;   // rows past the last one are never output
        }
        cnt[lm] = 0;
      }
      __syncthreads();  // lists and thresholds settled before the next tile's loads reuse LDS
      continue;
    }

    // 3. rare (heavy ties): some row has more passing values than slots.
    // Exact per-lane lists instead: each lane inserts its passing values into
    // a sorted list of 16; the lists of the two half-waves merge by shuffle
    // and one copy per wave goes to LDS ([0, WM): wave wv = 1, [WM, 2 WM):
    // wave wv = 0), where one thread per row merges them into the run's list.
    uint64_t* lists = reinterpret_cast<uint64_t*>(wm ? x1 : x0);
#pragma nounroll
    for (int j = 0; j < FJ; ++j) {
      const int lm = WM * wm + 32 * j + r;
      const int m = m0 + lm;
      const uint64_t tk = thrk[lm];
      const float tf = fresh ? thr[lm] : 0.f;
      const float tv = key_val(tk);
      const uint32_t tlo = uint32_t(tk);
      uint64_t L[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) L[q] = 0ull;
#pragma nounroll
      for (int hf = 0; hf < 2; ++hf) {
        float x[32];
        logits_half(2 * j + hf, x);
        const int base = lb + 64 * hf;   // vocabulary offset of x[0] in the tile
        uint32_t mask = pass_mask(x, base, hf, tf, tv, tlo, tk == 0ull);
        if (__builtin_amdgcn_ballot_w64(mask != 0u) != 0ull) {
          // stage the 32 values (lane-major) and visit the set bits
#pragma unroll
          for (int k = 0; k < 32; ++k) stg[k * WAVE + lane] = x[k];
          while (mask != 0u) {
            const int k = __builtin_ctz(mask);
            mask &= mask - 1u;
            const uint64_t key = rank_key(stg[k * WAVE + lane], uint32_t(n0 + base + voff(k)));
            if (key > L[15]) insert_key(L, key);
          }
        }
      }
      uint64_t brev[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) brev[q] = __shfl_xor(L[15 - q], 32, WAVE);
      bitonic_top<16>(L, brev);
      if (h == 0) {
        uint64_t* dst = lists + ((wv ? 0 : WM) + 32 * j + r) * 16;
#pragma unroll
        for (int q = 0; q < 16; ++q) dst[q] = L[q];
      }
    }
    __syncthreads();
    // each row's new candidates into the run's list (one thread per row;
    // rows with none keep their list)
    for (int lm = tid; lm < BM; lm += blockDim.x) {
      const int m = m0 + lm;
      const int half = lm / WM, lr = lm % WM;
      const uint64_t* ls = reinterpret_cast<const uint64_t*>(half ? x1 : x0);
      const bool any = ls[(WM + lr) * 16] != 0ull || ls[lr * 16] != 0ull;
      if (m < Mact && (any || fresh)) {
        uint64_t* o = p.cand + (int64_t(m) * p.runs + rg) * 16;
        uint64_t A[16], B[16], G[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) G[q] = fresh ? 0ull : o[15 - q];   // the run's list so far, reversed
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          A[q] = ls[(WM + lr) * 16 + q];
          B[q] = ls[lr * 16 + 15 - q];
        }
        bitonic_top<16>(A, B);
        bitonic_top<16>(A, G);
#pragma unroll
        for (int q = 0; q < 16; ++q) o[q] = A[q];
        thrk[lm] = A[15];
      } else if (m >= Mact) {
        thrk[lm] = ~0ull;   // rows past the last one are never output
      }
      cnt[lm] = 0;
    }
    __syncthreads();  // lists and thresholds settled before the next tile's loads reuse LDS
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {
struct LmPlan {
  int bm, nM, nN, runs, tpb;
};

// Row tile (256, 192 or 128 rows) and vocabulary runs: one block per CU
// (256 resident blocks), each sweeping tpb tiles; the choice minimises tpb
// times the relative cost of a tile against a 256-row one: 128-row tiles
// 0.6 (fp8) or 0.55 (bf16, whose 256-row tiles fit only two stage buffers
// in LDS and wait longer on the weight stream: measured 384 against 428 us
// at 240 x 151936 x 4096), 192-row tiles 0.78.  192-row tiles cover 384
// rows without padding, where 256-row tiles would compute 512.
// DFLASH2_LMHEAD_TILES_PER_BLOCK (1..64) overrides tpb, DFLASH2_LMHEAD_BM
// (128, 192 or 256) the row tile.
LmPlan lm_plan(int weight_dtype, int M, int V) {
  LmPlan best{};
  double best_cost = 1e300;
  int force = 0;
  if (const char* env = std::getenv("DFLASH2_LMHEAD_TILES_PER_BLOCK")) {
    const int v = std::atoi(env);
    if (v >= 1 && v <= 64) force = v;
  }
  int force_bm = 0;
  if (const char* env = std::getenv("DFLASH2_LMHEAD_BM")) {
    const int v = std::atoi(env);
    if (v == 128 || v == 192 || v == 256) force_bm = v;
  }
  for (int bm : {256, 192, 128}) {
    if (force_bm && bm != force_bm) continue;
    LmPlan pl;
    pl.bm = bm;
    pl.nM = (M + bm - 1) / bm;
    pl.nN = (V + kLBN - 1) / kLBN;
    const int runs_max = std::max(1, std::min(pl.nN, 256 / std::max(1, pl.nM)));
    pl.tpb = force ? std::min(force, pl.nN) : (pl.nN + runs_max - 1) / runs_max;
    pl.runs = (pl.nN + pl.tpb - 1) / pl.tpb;
    const double waves = double((int64_t(pl.nM) * pl.runs + 255) / 256);
    const double rel128 = weight_dtype == 1 ? 0.55 : 0.6;
    const double cost = waves * pl.tpb * (bm == 256 ? 1.0 : (bm == 192 ? 0.78 : rel128));
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = pl;
    }
  }
  return best;
}
}  // namespace

bool lmhead_tiled_ok(int weight_dtype, int M, int K, int k) {
  return weight_dtype != 0 && M > kTiledMinRows && K % kLKT == 0 && k <= 16;
}

int lmhead_tiled_lists(int weight_dtype, int M, int V) { return lm_plan(weight_dtype, M, V).runs; }

template <typename TW>
static void launch_lm_t(const LmTiledArgs& a, int bm, hipStream_t s) {
  const int blocks = a.nM * a.runs;
  const dim3 grid(unsigned((blocks + 7) / 8 * 8));
  // three stage buffers where they fit in LDS (not bf16 with 256 or 192 rows)
  constexpr int R256 = sizeof(TW) == 1 ? 3 : 2;
  if (bm == 256) hipLaunchKernelGGL((lmhead_tiled_kernel<TW, 256, R256>), grid, dim3(256), 0, s, a);
  else if (bm == 192) hipLaunchKernelGGL((lmhead_tiled_kernel<TW, 192, R256>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((lmhead_tiled_kernel<TW, 128, 3>), grid, dim3(256), 0, s, a);
}

void launch_lmhead_tiled(int weight_dtype, const LmHeadArgs& a, hipStream_t s) {
  const LmPlan pl = lm_plan(weight_dtype, a.M, a.N);
  LmTiledArgs t{};
  t.X = static_cast<const bf16_t*>(a.X); t.ldx = a.ldx;
  t.W = a.W; t.ldw = a.ldw; t.scale = a.scale;
  t.M = a.M; t.N = a.N; t.K = a.K; t.M_dev = a.M_dev; t.rs = a.rs;
  t.cand = a.cand; t.debug_logits = a.debug_logits;
  t.nM = pl.nM; t.runs = pl.runs; t.tpb = pl.tpb; t.nN = pl.nN;
  if (weight_dtype == 1) launch_lm_t<bf16_t>(t, pl.bm, s);
  else launch_lm_t<fp8_t>(t, pl.bm, s);
}

}  // namespace dfl

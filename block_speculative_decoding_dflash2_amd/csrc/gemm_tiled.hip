// Compute-bound GEMMs y = x * W^T for many activation rows (batched drafts):
// the linears and the lm_head of the batched and fp8 high-batch workloads,
// where every weight row meets hundreds of activation rows and the matrix
// cores, not HBM, set the pace.
//
// Block tile: BM = 128 activation rows x 256 weight rows, 4 waves; wave w
// owns weight rows [64 w, 64 w + 64) of the tile against all BM activation
// rows (acc = 2 x 4 MFMA 32x32x16 tiles, 64 float32 per lane), and two
// blocks share a CU.  The activation tile is shared by the four waves and
// goes through LDS (double buffered, 64 k per stage, rows padded to 144 bytes
// so 16-byte reads are conflict-free).  Weight rows are private to a wave:
// each wave fetches its 64 rows with coalesced loads one stage ahead into
// registers and copies them into its own LDS region, from which they are
// read in MFMA operand order.  fp8 weights are widened to bf16 when read
// from LDS (exact).
//
// Tiles are numbered with the activation tile fastest and dealt out so that
// each XCD (blocks go to the 8 XCDs round-robin) runs a contiguous run of
// tile numbers: the blocks that share a weight tile share that XCD's L2.
//
// Epilogues: float32 split-K partial sums (the same layout the
// weight-streaming kernels write, reduced by the consumer kernel), or with
// one K split the consumer itself (SwiGLU, or RoPE and the cache stores).
// The lm_head of many rows has its own kernel (lmhead_tiled.hip).
#include <algorithm>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace dfl {

namespace {
constexpr int kTBN = 256;            // weight rows per block (64 per wave)
constexpr int kTKT = 64;             // contraction depth per LDS stage
constexpr int kTXRow = kTKT * 2 + 16;  // LDS bytes per activation row
// Buffer resource word 3 for untyped 32-bit data on gfx9-family chips.
constexpr int kBufferFlags = 0x00020000;
}  // namespace

struct TiledArgs {
  const bf16_t* X; int64_t ldx;
  const void* W; int64_t ldw;
  const float* scale;
  int M, N, K;
  const int32_t* M_dev;
  RowScale rs;
  int splits, k_split;
  int groups;
  const void* Wg[kMaxGroups];
  const float* Sg[kMaxGroups];
  int64_t group_stride;
  float* P; int64_t ldp, split_stride;       // partial-sum epilogue
  int nM, nN, tiles;
  GemmEpi epi;                                // gemm_tiled_kernel consumer (one K split)
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Weight rows go through a wave-private LDS region: they are fetched with
// coalesced 16-byte loads (whole 128-byte row segments, 8 lanes per row for
// bf16) and read back in MFMA operand order.  Fetching them straight in
// operand order (32 rows x 32 bytes per instruction) runs at about a quarter
// of the L2 rate on this chip and starves the matrix cores.
template <typename TW> struct WLds;
template <> struct WLds<bf16_t> {
  static constexpr int ROWB = 144;   // 128 B of a stage + pad
  static constexpr int NLD = 8;      // coalesced 16-byte loads per lane per stage (8 rows x 128 B each)
  typedef u32x4 raw;
};
template <> struct WLds<fp8_t> {
  // 72-byte rows: the 8-byte operand reads of 32 consecutive rows then fall
  // on distinct banks (an 80-byte pitch maps rows r and r + 16 onto the same
  // banks; measured bank-conflict cycles were as many as the LDS busy cycles).
  // Rows are no longer 16-byte aligned, so they are written 8 bytes at a time.
  static constexpr int ROWB = 72;
  static constexpr int NLD = 4;      // 16 rows x 64 B each
  typedef u32x4 raw;
};

// Main loop on v_mfma_f32_32x32x16_bf16: D[32 x 32] += A[32 x 16] B[16 x 32],
// lane l supplying row l % 32 of A (a weight row) and column l % 32 of B (an
// activation row) with the 8 contraction indices 8 (l / 32) .. + 7 of a
// 16-wide k step.  Output: lane l holds D[8 q + 4 (l / 32) + e][l % 32] in
// element 4 q + e.
template <typename TW, int FM>
struct TiledMain {
  static constexpr int BM = 16 * FM;
  static constexpr int F2 = BM / 32;
  static constexpr int XQ = BM / 32;
  static constexpr int XBUF = BM * kTXRow;
  static constexpr int WBUF = 64 * WLds<TW>::ROWB;   // per wave
  static constexpr int LDS_BYTES = 2 * XBUF + 4 * WBUF;

  // acc[i][j]: lane (r, h) holds y[n0w + 32 i + 8 q + 4 h + e][m0 + 32 j + r]
  // in element 4 q + e, summed over k in [kb, kb + 64 nk).  Rows past the
  // operands' ends are clamped to the last row (their results are never
  // stored); loads past the last stage repeat the last stage, so the loads
  // in flight are the same on every pass of the loop and the compiler's
  // wait counts stay exact.
  __device__ static void run(const bf16_t* __restrict__ X, int64_t ldx, const TW* __restrict__ W,
                             int64_t ldw, int N, int Mact, int n0w, int m0, int kb, int nk,
                             f32x16 (&acc)[2][F2], char* lds) {
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid >> 6;
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < F2; ++j) acc[i][j] = f32x16{};
    if (nk <= 0) return;
    constexpr int SW = int(sizeof(TW));
    constexpr int WROWB = WLds<TW>::ROWB, NLD = WLds<TW>::NLD;
    constexpr int LPR = 64 * SW / 16;          // lanes per row in a coalesced load (8 bf16, 4 fp8)
    constexpr int RPI = 64 / LPR;              // rows per load instruction
    const int xr = tid >> 3, xc = tid & 7;
    // 64-bit bases at the first row of the wave's weight rows and of the
    // block's activation rows (and at k = kb); the per-lane offsets from
    // them stay below 2^32 bytes because a tile spans at most 128 rows of at
    // most 2^20 elements (both checked when the handle is created)
    const int wb0 = min(n0w, N - 1), xb0 = min(m0, Mact - 1);
    const char* wbase = reinterpret_cast<const char*>(W) + (int64_t(wb0) * ldw + kb) * SW;
    const char* xbase = reinterpret_cast<const char*>(X) + (int64_t(xb0) * ldx + kb) * 2;
    // coalesced weight loads: instruction q covers rows RPI q .. RPI q + RPI - 1 of the wave's 64
    const int wrow = lane / LPR, wcol = lane % LPR;
    uint32_t woffc[NLD], xoffc[XQ];
#pragma unroll
    for (int q = 0; q < NLD; ++q)
      woffc[q] = uint32_t(min(n0w + RPI * q + wrow, N - 1) - wb0) * uint32_t(ldw) * SW + uint32_t(16 * wcol);
#pragma unroll
    for (int q = 0; q < XQ; ++q)
      xoffc[q] = (uint32_t(min(m0 + xr + 32 * q, Mact - 1) - xb0) * uint32_t(ldx) + uint32_t(8 * xc)) * 2u;
    char* xdst = lds + xr * kTXRow + 16 * xc;
    const char* xsrc = lds + r * kTXRow + 16 * h;
    char* wl = lds + 2 * XBUF + wave * WBUF;
    char* wdst = wl + wrow * WROWB + 16 * wcol;
    const char* wsrc = wl + r * WROWB + 8 * SW * h;
    u32x4 wr[NLD];
    u32x4 xs[XQ];
    auto load_w = [&](int kt) {
#pragma unroll
      for (int q = 0; q < NLD; ++q) wr[q] = *reinterpret_cast<const u32x4*>(wbase + woffc[q] + uint32_t(kt * kTKT * SW));
    };
    auto store_w = [&]() {
#pragma unroll
      for (int q = 0; q < NLD; ++q) {
        char* d = wdst + q * RPI * WROWB;
        if constexpr (WROWB % 16 == 0) {
          *reinterpret_cast<u32x4*>(d) = wr[q];
        } else {
          *reinterpret_cast<u32x2*>(d) = u32x2{wr[q][0], wr[q][1]};
          *reinterpret_cast<u32x2*>(d + 8) = u32x2{wr[q][2], wr[q][3]};
        }
      }
    };
    auto load_x = [&](int kt) {
#pragma unroll
      for (int q = 0; q < XQ; ++q) xs[q] = *reinterpret_cast<const u32x4*>(xbase + xoffc[q] + uint32_t(kt * kTKT * 2));
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int q = 0; q < XQ; ++q)
        *reinterpret_cast<u32x4*>(xdst + buf * XBUF + q * 32 * kTXRow) = xs[q];
    };
    auto compute = [&](int buf) {
      __builtin_amdgcn_s_setprio(1);  // the wave with matrix work ready issues first
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag8Bf16 wf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const char* p = wsrc + i * 32 * WROWB + s * 16 * SW;
          if (SW == 2) wf[i].v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
          else fp8x8_to_frag(wf[i], *reinterpret_cast<const u32x2*>(p));
        }
#pragma unroll
        for (int j = 0; j < F2; ++j) {
          bf16x8 xf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                xsrc + buf * XBUF + j * 32 * kTXRow + 32 * s));
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i].v, xf, acc[i][j], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // W(kt) sits in registers at the start of stage kt and is copied to this
    // wave's LDS region; X(kt) is in LDS buffer kt & 1.
    load_w(0);
    load_x(0);
    store_x(0);
    load_x(min(1, nk - 1));
    __syncthreads();
    auto stage = [&](int buf, int kt) {
      store_w();
      __builtin_amdgcn_sched_barrier(0);
      load_w(min(kt + 1, nk - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(buf);
      __builtin_amdgcn_sched_barrier(0);
      store_x(buf ^ 1);
      load_x(min(kt + 2, nk - 1));
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + 2 <= nk; kt += 2) {
      stage(0, kt);
      stage(1, kt + 1);
    }
    if (kt < nk) stage(0, kt);
  }
};

// Logical tile of this block; false for padding blocks.
__device__ __forceinline__ bool tiled_tile(const TiledArgs& p, int& mt, int& nt, int& split, int& group) {
  const int per = gridDim.x >> 3;  // the grid is a multiple of 8
  const int t = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (t >= p.tiles) return false;
  mt = t % p.nM;
  int rest = t / p.nM;
  nt = rest % p.nN;
  rest /= p.nN;
  split = rest % p.splits;
  group = rest / p.splits;
  return true;
}

// 1 / rms of activation rows [m0, m0 + BM) into LDS (rows past Mact: 1).
template <int BM>
__device__ __forceinline__ void tiled_row_scales(const RowScale& rs, int m0, int Mact, float* inv) {
  for (int t = threadIdx.x; t < BM; t += blockDim.x) {
    float v = 1.f;
    const int m = m0 + t;
    if (rs.sumsq && m < Mact) {
      float s = 0.f;
      for (int c = 0; c < rs.blocks; ++c) s += rs.sumsq[int64_t(m) * rs.blocks + c];
      v = 1.0f / sqrtf(s * rs.inv_width + rs.eps);
    }
    inv[t] = v;
  }
}

// Partial sums: P[group][split][m][n] = inv_rms[m] * scale[n] * sum_k x[m][k] W[n][k],
// or (one K split, EPI != EPI_NONE) that value's consumer applied in place:
//  * EPI_SWIGLU: block nt holds gate rows [128 nt, 128 nt + 128) in waves 0-1
//    and the matching up rows F + ... in waves 2-3; the up values go through
//    LDS and waves 0-1 write SiLU(gate) * up;
//  * EPI_QKV: the tile's columns are whole heads (d = 64 or 128); RoPE pairs
//    (c, c + d/2) sit in one lane (d = 64) or in waves 2k and 2k + 1
//    (d = 128, the odd wave's values go through LDS); q heads go to q_out,
//    k and v heads to this layer's cache rows.
// BM = 128 fits in 256 registers per lane, so two blocks share a CU and
// cover each other's load latency.
template <typename TW, int FM, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_tiled_kernel(TiledArgs p) {
  typedef TiledMain<TW, FM> Main;
  constexpr int BM = Main::BM, F2 = Main::F2;
  constexpr int EB = EPI == EPI_NONE ? 0 : BM * 132 * 4;  // exchange buffer [BM][132] floats
  __shared__ __attribute__((aligned(16))) char lds[Main::LDS_BYTES > EB ? Main::LDS_BYTES : EB];
  __shared__ float inv[BM];
  __shared__ double inv_freq[EPI == EPI_QKV ? 64 : 1];
  int mt, nt, split, group;
  if (!tiled_tile(p, mt, nt, split, group)) return;
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m0 = mt * BM;
  if (m0 >= Mact) return;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const int r = lane & 31, h = lane >> 5;
  int n0w = nt * kTBN + 64 * wave;
  if (EPI == EPI_SWIGLU) n0w = (wave < 2 ? 0 : p.epi.F) + 128 * nt + 64 * (wave & 1);
  const TW* W = static_cast<const TW*>(p.groups > 1 ? p.Wg[group] : p.W);
  const float* scale = p.groups > 1 ? p.Sg[group] : p.scale;
  const int kb = split * p.k_split;
  const int nk = (min(p.K, kb + p.k_split) - kb) / kTKT;
  tiled_row_scales<BM>(p.rs, m0, Mact, inv);  // visible after the main loop's barriers
  if (EPI == EPI_QKV && threadIdx.x < p.epi.d / 2)
    inv_freq[threadIdx.x] = pow(double(p.epi.theta), -2.0 * double(threadIdx.x) / double(p.epi.d));
  f32x16 acc[2][F2];
  Main::run(p.X, p.ldx, W, p.ldw, p.N, Mact, n0w, m0, kb, nk, acc, lds);
  __syncthreads();
  // lane (r, h) holds y[n0w + 32 i + 8 q + 4 h + e][m0 + 32 j + r] in acc[i][j][4 q + e];
  // scale it to the stored value
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nb = n0w + 32 * i + 8 * q + 4 * h;
      float s[4] = {1.f, 1.f, 1.f, 1.f};
      if (scale) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = scale[min(nb + e, p.N - 1)];
      }
#pragma unroll
      for (int j = 0; j < F2; ++j) {
        const float iv = inv[32 * j + r];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = (acc[i][j][4 * q + e] * s[e]) * iv;
      }
    }
  }
  if (EPI == EPI_NONE) {
    float* P = p.P + int64_t(group) * p.group_stride + int64_t(split) * p.split_stride;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nb = n0w + 32 * i + 8 * q + 4 * h;
        if (nb >= p.N) continue;
#pragma unroll
        for (int j = 0; j < F2; ++j) {
          const int m = m0 + 32 * j + r;
          if (m >= Mact) continue;
          const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          float* dst = P + int64_t(m) * p.ldp + nb;
          if (nb + 3 < p.N && (p.ldp & 3) == 0) {
            *reinterpret_cast<f32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nb + e < p.N) dst[e] = v[e];
          }
        }
      }
    }
    return;
  }
  // exchange: waves 2-3 (up rows, or the second half of each 128-wide head)
  // publish their values at [row][column within the pair of waves]
  float* xb = reinterpret_cast<float*>(lds);
  const bool second = EPI == EPI_SWIGLU ? wave >= 2 : (p.epi.d == 128 && (wave & 1));
  const bool exchange = EPI == EPI_SWIGLU || p.epi.d == 128;
  if (exchange && second) {
    const int cw = EPI == EPI_SWIGLU ? 64 * (wave & 1) : 64 * (wave >> 1);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < F2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          xb[(32 * j + r) * 132 + cw + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3)] = acc[i][j][v];
  }
  __syncthreads();
  if (exchange && second) return;
  const int cw = EPI == EPI_SWIGLU ? 64 * (wave & 1) : 64 * (wave >> 1);
  if (EPI == EPI_SWIGLU) {
    const int F = p.epi.F;
    bf16_t* out = static_cast<bf16_t*>(p.epi.act_out);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = 128 * nt + 64 * (wave & 1) + 32 * i + 8 * q + 4 * h;
#pragma unroll
        for (int j = 0; j < F2; ++j) {
          const int m = m0 + 32 * j + r;
          if (m >= Mact) continue;
          uint32_t o[2];
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            float y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float gt = acc[i][j][4 * q + e + u];
              const float up = xb[(32 * j + r) * 132 + cw + 32 * i + 8 * q + 4 * h + e + u];
              y[u] = gt / (1.0f + expf(-gt)) * up;
            }
            o[e / 2] = uint32_t(f32_to_bf16(y[0])) | (uint32_t(f32_to_bf16(y[1])) << 16);
          }
          bf16_t* dst = out + int64_t(m) * F + f;
          if (f + 3 < F && (F & 3) == 0) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{o[0], o[1]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (f + e < F) dst[e] = bf16_t(o[e / 2] >> (16 * (e & 1)));
          }
        }
      }
    return;
  }
  // EPI_QKV: this lane's columns c (first half of a head) pair with c + d/2
  const GemmEpi& e = p.epi;
  const int d = e.d, half = d / 2, nh = e.nq + 2 * e.nkv;
  bf16_t* qo = static_cast<bf16_t*>(e.q_out);
  bf16_t* kc = static_cast<bf16_t*>(e.k_layer);
  bf16_t* vc = static_cast<bf16_t*>(e.v_layer);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (d == 64 && i == 1) continue;  // d = 64: the pair is (i = 0, i = 1) of this lane
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c0 = n0w + 32 * i + 8 * q + 4 * h;  // output column of the first element
      const int head = c0 / d, ci = c0 % d;          // ci < d/2
      if (head >= nh) continue;
#pragma unroll
      for (int j = 0; j < F2; ++j) {
        const int m = m0 + 32 * j + r;
        if (m >= Mact) continue;
        const int b = m / e.bs, t = m % e.bs;
        const int pos = e.ctx_lens[b] + t;
        float y0[4], y1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float x0 = acc[i][j][4 * q + u];
          const float x1 = d == 64 ? acc[1][j][4 * q + u]
                                   : xb[(32 * j + r) * 132 + cw + 32 * i + 8 * q + 4 * h + u];
          if (head < e.nq + e.nkv) {
            // angle in double, reduced to [-pi, pi], then float sine and cosine
            const double ang = double(pos) * inv_freq[ci + u];
            const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
            float sn, cs;
            sincosf(float(red), &sn, &cs);
            y0[u] = x0 * cs - x1 * sn;
            y1[u] = x1 * cs + x0 * sn;
          } else {
            y0[u] = x0;
            y1[u] = x1;
          }
        }
        const u32x2 lo = {uint32_t(f32_to_bf16(y0[0])) | (uint32_t(f32_to_bf16(y0[1])) << 16),
                          uint32_t(f32_to_bf16(y0[2])) | (uint32_t(f32_to_bf16(y0[3])) << 16)};
        const u32x2 hi = {uint32_t(f32_to_bf16(y1[0])) | (uint32_t(f32_to_bf16(y1[1])) << 16),
                          uint32_t(f32_to_bf16(y1[2])) | (uint32_t(f32_to_bf16(y1[3])) << 16)};
        if (head < e.nq) {
          bf16_t* dst = qo + (int64_t(m) * e.nq + head) * d;
          *reinterpret_cast<u32x2*>(dst + ci) = lo;
          *reinterpret_cast<u32x2*>(dst + ci + half) = hi;
        } else if (pos >= 0 && pos < e.Lmax) {
          if (head < e.nq + e.nkv) {
            const int g = head - e.nq;
            bf16_t* dst = kc + ((int64_t(b) * e.nkv + g) * e.Lmax + pos) * d;
            *reinterpret_cast<u32x2*>(dst + ci) = lo;
            *reinterpret_cast<u32x2*>(dst + ci + half) = hi;
          } else {
            const int g = head - e.nq - e.nkv;
            bf16_t* dst = vc + (int64_t(b) * e.nkv + g) * d * e.Lmax + pos;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              dst[int64_t(ci + u) * e.Lmax] = f32_to_bf16(y0[u]);
              dst[int64_t(ci + half + u) * e.Lmax] = f32_to_bf16(y1[u]);
            }
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int tiled_block_rows(int M) {
  (void)M;
  return 128;
}

bool gemm_tiled_ok(int weight_dtype, int M, int K) {
  return weight_dtype != 0 && M > kTiledMinRows && K % kTKT == 0;
}
template <typename TW>
static void launch_tiled_t(const TiledArgs& t, hipStream_t s) {
  const dim3 grid(unsigned((t.tiles + 7) / 8 * 8));
  if (t.epi.kind == EPI_SWIGLU) hipLaunchKernelGGL((gemm_tiled_kernel<TW, 8, EPI_SWIGLU>), grid, dim3(256), 0, s, t);
  else if (t.epi.kind == EPI_QKV) hipLaunchKernelGGL((gemm_tiled_kernel<TW, 8, EPI_QKV>), grid, dim3(256), 0, s, t);
  else hipLaunchKernelGGL((gemm_tiled_kernel<TW, 8, EPI_NONE>), grid, dim3(256), 0, s, t);
}

bool tiled_epi_fusable(const GemmArgs& a) {
  if (a.epi.kind == EPI_NONE || a.splits != 1 || a.groups > 1 || a.M_dev) return false;
  if (a.epi.kind == EPI_SWIGLU) return a.N == 2 * a.epi.F && a.epi.act_out;
  if (a.epi.kind == EPI_QKV) return (a.epi.d == 64 || a.epi.d == 128) && a.N % a.epi.d == 0;
  return false;
}

void launch_gemm_tiled(int weight_dtype, const GemmArgs& a, hipStream_t s) {
  TiledArgs t{};
  t.X = static_cast<const bf16_t*>(a.X); t.ldx = a.ldx;
  t.W = a.W; t.ldw = a.ldw; t.scale = a.scale;
  t.M = a.M; t.N = a.N; t.K = a.K; t.M_dev = a.M_dev; t.rs = a.rs;
  t.splits = a.splits; t.k_split = a.k_split;
  t.groups = a.groups > 1 ? a.groups : 1;
  for (int i = 0; i < kMaxGroups; ++i) { t.Wg[i] = a.Wg[i]; t.Sg[i] = a.Sg[i]; }
  t.group_stride = a.group_stride;
  t.P = a.P; t.ldp = a.ldp; t.split_stride = a.split_stride;
  t.epi = a.epi;
  if (!tiled_epi_fusable(a)) t.epi.kind = EPI_NONE;
  t.nM = (a.M + tiled_block_rows(a.M) - 1) / tiled_block_rows(a.M);
  t.nN = t.epi.kind == EPI_SWIGLU ? (a.epi.F + 127) / 128 : (a.N + kTBN - 1) / kTBN;
  t.tiles = t.nM * t.nN * t.splits * t.groups;
  if (weight_dtype == 1) launch_tiled_t<bf16_t>(t, s);
  else launch_tiled_t<fp8_t>(t, s);
}

}  // namespace dfl

// Compute-bound GEMMs y = x * W^T for many activation rows (batched drafts):
// the linears and the lm_head of the batched and fp8 high-batch workloads,
// where every weight row meets hundreds of activation rows and the matrix
// cores, not HBM, set the pace.
//
// Block tile: BM = 16 * FM activation rows x 256 weight rows, 4 waves; wave w
// owns weight rows [64 w, 64 w + 64) of the tile against all BM activation
// rows (acc = 2 x BM/32 MFMA 32x32x16 tiles, BM/2 float32 per lane).  The
// activation tile is shared by the four waves and goes through LDS (double
// buffered, 64 k per stage, rows padded to 144 bytes so 16-byte reads are
// conflict-free).  Weight fragments are private to a wave, so they are read
// straight from global memory into MFMA operand registers (one stage ahead)
// and never touch LDS, which halves LDS traffic against staging both
// operands.  fp8 weights are widened to bf16 in registers (exact).
//
// Tiles are numbered with the activation tile fastest and dealt out so that
// each XCD (blocks go to the 8 XCDs round-robin) runs a contiguous run of
// tile numbers: the blocks that share a weight tile share that XCD's L2.
//
// Two epilogues: float32 split-K partial sums (the same layout the
// weight-streaming kernels write, reduced by the consumer kernel), and the
// lm_head's per-256-vocabulary-group top-k (see the top-k section below).
#include "common.h"
#include "kernels.h"

namespace dfl {

namespace {
constexpr int kTBN = 256;            // weight rows per block (64 per wave)
constexpr int kTKT = 64;             // contraction depth per LDS stage
constexpr int kTXRow = kTKT * 2 + 16;  // LDS bytes per activation row
constexpr int kTSlots = 32;          // top-k candidate slots per row and round
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
  int k, vgroups; uint64_t* cand; float* debug_logits;  // top-k epilogue
  int nM, nN, tiles;
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Main loop on v_mfma_f32_32x32x16_bf16: D[32 x 32] += A[32 x 16] B[16 x 32],
// lane l supplying row l % 32 of A (a weight row) and column l % 32 of B (an
// activation row) with the 8 contraction indices 8 (l / 32) .. + 7 of a
// 16-wide k step.  Output: lane l holds D[8 q + 4 (l / 32) + e][l % 32] in
// element 4 q + e.
template <typename TW, int FM>
struct TiledMain {
  static constexpr int BM = 16 * FM;
  static constexpr int F2 = BM / 32;  // 32-row activation fragments
  static constexpr int XQ = BM / 32;  // 16-byte activation loads per thread per stage
  static constexpr int XBUF = BM * kTXRow;
  typedef typename WFrag<TW>::raw WRaw;

  // acc[i][j]: lane (r, h) holds y[n0w + 32 i + 8 q + 4 h + e][m0 + 32 j + r]
  // in element 4 q + e, summed over k in [kb, kb + 64 nk).  Tile 1 is fetched
  // unconditionally (tile 0 again when nk == 1) so the loads in flight at
  // the loop entry match those at its back edge and the compiler's wait
  // counts stay exact.
  __device__ static void run(const bf16_t* __restrict__ X, int64_t ldx, const TW* __restrict__ W,
                             int64_t ldw, int N, int Mact, int n0w, int m0, int kb, int nk,
                             f32x16 (&acc)[2][F2], char* lds) {
    const int tid = threadIdx.x, lane = tid & (WAVE - 1);
    const int r = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < F2; ++j) acc[i][j] = f32x16{};
    if (nk <= 0) return;
    const TW* wp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = min(n0w + 32 * i + r, N - 1);
      wp[i] = W + int64_t(n) * ldw + kb + 8 * h;
    }
    const int xr = tid >> 3, xc = tid & 7;
    const bf16_t* xp[XQ];
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int m = min(m0 + xr + 32 * q, Mact - 1);
      xp[q] = X + int64_t(m) * ldx + kb + 8 * xc;
    }
    char* xdst = lds + xr * kTXRow + 16 * xc;
    const char* xsrc = lds + r * kTXRow + 16 * h;
    WRaw wr[2][4][2];
    u32x4 xs[XQ];

    auto load_w = [&](int st, int kt) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i) wr[st][s][i] = WFrag<TW>::load(wp[i] + kt * kTKT + 16 * s);
    };
    auto load_x = [&](int kt) {
#pragma unroll
      for (int q = 0; q < XQ; ++q) xs[q] = *reinterpret_cast<const u32x4*>(xp[q] + kt * kTKT);
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int q = 0; q < XQ; ++q)
        *reinterpret_cast<u32x4*>(xdst + buf * XBUF + q * 32 * kTXRow) = xs[q];
    };
    auto compute = [&](int st, int buf) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        Frag8Bf16 wf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) WFrag<TW>::cvt(wf[i], wr[st][s][i]);
#pragma unroll
        for (int j = 0; j < F2; ++j) {
          bf16x8 xf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                xsrc + buf * XBUF + j * 32 * kTXRow + 32 * s));
#pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i].v, xf, acc[i][j], 0, 0, 0);
        }
      }
    };
    load_x(0);
    load_w(0, 0);
    store_x(0);
    const int k1 = nk > 1 ? 1 : 0;
    load_x(k1);
    load_w(1, k1);
    __syncthreads();
    int kt = 0;
    for (; kt + 4 <= nk; kt += 2) {
      compute(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      store_x(1);
      load_x(kt + 2);
      load_w(0, kt + 2);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      compute(1, 1);
      __builtin_amdgcn_sched_barrier(0);
      store_x(0);
      load_x(kt + 3);
      load_w(1, kt + 3);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    const int rem = nk - kt;
    compute(0, 0);
    if (rem >= 2) {
      store_x(1);
      if (rem == 3) {
        load_x(kt + 2);
        load_w(0, kt + 2);
      }
      __syncthreads();
      compute(1, 1);
      if (rem == 3) {
        store_x(0);
        __syncthreads();
        compute(0, 0);
      }
    }
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

// Partial sums: P[group][split][m][n] = inv_rms[m] * scale[n] * sum_k x[m][k] W[n][k].
template <typename TW, int FM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_tiled_kernel(TiledArgs p) {
  typedef TiledMain<TW, FM> Main;
  constexpr int BM = Main::BM, F2 = Main::F2;
  __shared__ __attribute__((aligned(16))) char lds[2 * Main::XBUF];
  __shared__ float inv[BM];
  int mt, nt, split, group;
  if (!tiled_tile(p, mt, nt, split, group)) return;
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m0 = mt * BM;
  if (m0 >= Mact) return;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const int r = lane & 31, h = lane >> 5;
  const int n0w = nt * kTBN + 64 * wave;
  const TW* W = static_cast<const TW*>(p.groups > 1 ? p.Wg[group] : p.W);
  const float* scale = p.groups > 1 ? p.Sg[group] : p.scale;
  const int kb = split * p.k_split;
  const int nk = (min(p.K, kb + p.k_split) - kb) / kTKT;
  tiled_row_scales<BM>(p.rs, m0, Mact, inv);  // visible after the main loop's barriers
  f32x16 acc[2][F2];
  Main::run(p.X, p.ldx, W, p.ldw, p.N, Mact, n0w, m0, kb, nk, acc, lds);
  __syncthreads();
  float* P = p.P + int64_t(group) * p.group_stride + int64_t(split) * p.split_stride;
  // lane (r, h) holds y[n0w + 32 i + 8 q + 4 h + e][m0 + 32 j + r] in acc[i][j][4 q + e]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nb = n0w + 32 * i + 8 * q + 4 * h;
      if (nb >= p.N) continue;
      float s[4] = {1.f, 1.f, 1.f, 1.f};
      if (scale) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = scale[min(nb + e, p.N - 1)];
      }
#pragma unroll
      for (int j = 0; j < F2; ++j) {
        const int m = m0 + 32 * j + r;
        if (m >= Mact) continue;
        const float iv = inv[32 * j + r];
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (acc[i][j][4 * q + e] * s[e]) * iv;
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
}

// ---------------------------------------------------------------------------
// lm_head + top-k.  Each block ranks its 256 vocabulary ids for each of its
// BM rows and writes the row's k best keys (value desc, id asc) for that
// vocabulary group, the same candidate layout the weight-streaming lm_head
// writes; the merge kernel then picks each row's final k.
//
// Selecting 16 of 256 values per row cheaply:
//  1. a lane holds 32 values of each of its rows, in two groups of 16 (one
//     per 32-row weight fragment); it keeps the largest and second largest
//     of each group.  The row's 16 groups give 32 such values, and their
//     16th largest, T, has at least 16 of the row's values >= T, so no
//     value below T can be among the row's top 16;
//  2. values >= T (typically ~18 of 256) are appended to the row's candidate
//     slots in LDS; the thread owning the row insertion-sorts them into a
//     register list of 16 keys;
//  3. if a row had more than kTSlots values >= T, another round takes the
//     values not yet appended whose key beats the row's current 16th key.
// ---------------------------------------------------------------------------
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

__device__ __forceinline__ void insert16(uint64_t (&L)[16], uint64_t x) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool c = x > L[i];
    const uint64_t t = L[i];
    L[i] = c ? x : t;
    x = c ? t : x;
  }
}

template <typename TW, int FM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void lmhead_tiled_kernel(TiledArgs p) {
  typedef TiledMain<TW, FM> Main;
  constexpr int BM = Main::BM, F2 = Main::F2;
  constexpr int XB = 2 * Main::XBUF;
  constexpr int CB = BM * kTSlots * 8;
  constexpr int LB = XB > CB ? XB : CB;
  __shared__ __attribute__((aligned(16))) char lds[LB];
  __shared__ float inv[BM];
  __shared__ float thr[BM];
  __shared__ uint64_t thrk[BM];
  __shared__ int cnt[BM];
  int mt, nt, split, group;
  if (!tiled_tile(p, mt, nt, split, group)) return;
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m0 = mt * BM;
  if (m0 >= Mact) return;
  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid & (WAVE - 1);
  const int r = lane & 31, h = lane >> 5;
  const int n0w = nt * kTBN + 64 * wave;
  tiled_row_scales<BM>(p.rs, m0, Mact, inv);
  f32x16 acc[2][F2];
  Main::run(p.X, p.ldx, static_cast<const TW*>(p.W), p.ldw, p.N, Mact, n0w, m0, 0, p.K / kTKT, acc, lds);
  __syncthreads();  // every wave is done with the activation stages

  // logits (the same float32 steps as the weight-streaming lm_head); value
  // v = 4 q + e of acc[i][j] is vocabulary id n0w + 32 i + 8 q + 4 h + e of
  // row m0 + 32 j + r
  float* ab = reinterpret_cast<float*>(lds);  // [BM][33]: per-group top-2 of each row
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    float s[16];
#pragma unroll
    for (int v = 0; v < 16; ++v)
      s[v] = p.scale ? p.scale[min(n0w + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3), p.N - 1)] : 1.f;
#pragma unroll
    for (int j = 0; j < F2; ++j) {
      const float iv = inv[32 * j + r];
      const int m = m0 + 32 * j + r;
      float a = -INFINITY, b = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = acc[i][j][v];
        x *= s[v];
        x *= iv;
        x = x + 0.0f;
        acc[i][j][v] = x;
        const bool valid = n0w + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3) < p.N;
        const float y = valid ? x : -INFINITY;
        b = fmaxf(b, fminf(a, y));
        a = fmaxf(a, y);
      }
      if (p.debug_logits && m < Mact) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nb = n0w + 32 * i + 8 * q + 4 * h;
          float* dst = p.debug_logits + int64_t(m) * p.N + nb;
          if (nb + 3 < p.N && (p.N & 3) == 0) {
            *reinterpret_cast<f32x4*>(dst) =
                f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (nb + e < p.N) dst[e] = acc[i][j][4 * q + e];
          }
        }
      }
      const int slot = ((wave * 2 + h) * 2 + i) * 2;
      ab[(32 * j + r) * 33 + slot] = a;
      ab[(32 * j + r) * 33 + slot + 1] = b;
    }
  }
  __syncthreads();
  if (tid < BM) {
    float A[16], B[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      A[q] = ab[tid * 33 + 2 * q];
      B[q] = ab[tid * 33 + 2 * q + 1];
    }
    sort16_desc(A);
    sort16_desc(B);
    // the 16 largest of the union are max(A[q], B[15 - q]); T is their minimum
    float T = INFINITY;
#pragma unroll
    for (int q = 0; q < 16; ++q) T = fminf(T, fmaxf(A[q], B[15 - q]));
    thr[tid] = T;
    thrk[tid] = ~0ull;
    cnt[tid] = 0;
  }
  __syncthreads();  // ab is dead from here; its space holds the candidate slots
  uint64_t* slots = reinterpret_cast<uint64_t*>(lds);
  uint32_t sub[F2] = {};  // values already appended: bit 16 i + v of row fragment j
  uint64_t list[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) list[q] = 0ull;
  for (int round = 0;; ++round) {
#pragma unroll
    for (int j = 0; j < F2; ++j) {
      const int row = 32 * j + r;
      const float tf = thr[row];
      const uint64_t tk = thrk[row];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int n = n0w + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          const uint32_t bit = 1u << (16 * i + v);
          const float x = acc[i][j][v];
          bool pass = n < p.N && !(sub[j] & bit);
          if (round == 0) pass = pass && x >= tf;
          else pass = pass && rank_key(x, uint32_t(n)) > tk;
          if (pass) {
            const int sl = atomicAdd(&cnt[row], 1);
            if (sl < kTSlots) {
              slots[row * kTSlots + sl] = rank_key(x, uint32_t(n));
              sub[j] |= bit;
            }
          }
        }
      }
    }
    __syncthreads();
    bool more = false;
    if (tid < BM) {
      const int c = cnt[tid];
      const int nn = min(c, kTSlots);
      for (int q = 0; q < nn; ++q) insert16(list, slots[tid * kTSlots + q]);
      more = c > kTSlots;
      thrk[tid] = more ? list[15] : ~0ull;
      cnt[tid] = 0;
    }
    if (!__syncthreads_or(more)) break;
  }
  if (tid < BM && m0 + tid < Mact) {
    uint64_t* out = p.cand + (int64_t(m0 + tid) * p.vgroups + nt) * p.k;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (q < p.k) out[q] = list[q];
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int tiled_fm(int M) { return M <= 128 ? 8 : 16; }
int tiled_block_rows(int M) { return 16 * tiled_fm(M); }

bool gemm_tiled_ok(int weight_dtype, int M, int K) {
  return weight_dtype != 0 && M > kTiledMinRows && K % kTKT == 0;
}
bool lmhead_tiled_ok(int weight_dtype, int M, int K, int k) {
  return gemm_tiled_ok(weight_dtype, M, K) && k <= 16;
}

// The lm_head's top-k epilogue keeps every logit of the tile in registers
// while it ranks them; at BM = 256 that does not fit, so it runs at BM = 128.
int lmhead_tiled_block_rows() { return 128; }

template <typename TW>
static void launch_tiled_t(const TiledArgs& t, bool topk, hipStream_t s) {
  const dim3 grid(unsigned((t.tiles + 7) / 8 * 8));
  if (topk) hipLaunchKernelGGL((lmhead_tiled_kernel<TW, 8>), grid, dim3(256), 0, s, t);
  else if (tiled_fm(t.M) == 8) hipLaunchKernelGGL((gemm_tiled_kernel<TW, 8>), grid, dim3(256), 0, s, t);
  else hipLaunchKernelGGL((gemm_tiled_kernel<TW, 16>), grid, dim3(256), 0, s, t);
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
  t.nM = (a.M + tiled_block_rows(a.M) - 1) / tiled_block_rows(a.M);
  t.nN = (a.N + kTBN - 1) / kTBN;
  t.tiles = t.nM * t.nN * t.splits * t.groups;
  if (weight_dtype == 1) launch_tiled_t<bf16_t>(t, false, s);
  else launch_tiled_t<fp8_t>(t, false, s);
}

void launch_lmhead_tiled(int weight_dtype, const LmHeadArgs& a, hipStream_t s) {
  TiledArgs t{};
  t.X = static_cast<const bf16_t*>(a.X); t.ldx = a.ldx;
  t.W = a.W; t.ldw = a.ldw; t.scale = a.scale;
  t.M = a.M; t.N = a.N; t.K = a.K; t.M_dev = a.M_dev; t.rs = a.rs;
  t.splits = 1; t.k_split = a.K; t.groups = 1;
  t.k = a.k; t.vgroups = a.groups; t.cand = a.cand; t.debug_logits = a.debug_logits;
  t.nM = (a.M + lmhead_tiled_block_rows() - 1) / lmhead_tiled_block_rows();
  t.nN = (a.N + kTBN - 1) / kTBN;
  t.tiles = t.nM * t.nN;
  if (weight_dtype == 1) launch_tiled_t<bf16_t>(t, true, s);
  else launch_tiled_t<fp8_t>(t, true, s);
}

}  // namespace dfl

// Weight-streaming GEMMs y = x * W^T on the gfx950 matrix cores.
//
// Every linear of the draft (feature projection, QKV, O, gate/up, down) and
// the lm_head multiplies a few activation rows (B * block_size) by a large
// weight.  With few rows the work is bound by reading the weight once from
// HBM.  Each wave owns 16*RT weight rows and a K range and walks it in
// groups of 256 bytes per row.  A group is loaded with non-temporal 16-byte
// loads in which each quarter-wave reads 256 contiguous bytes of one row (4
// rows per instruction); on this chip that pattern streams ~37% faster than
// loading straight into the MFMA operand layout (16 rows x 64 bytes per
// instruction).  The group then goes through a wave-private LDS tile (rows
// padded to 272 bytes, conflict-free) and is read back as MFMA operands.
// Loads run NSG groups ahead of the math in a ring of register stages.
//
// Activation operands: with at most 16 activation rows (bf16 activations)
// the block first copies its rows' K range of the activations into LDS
// (global-to-LDS loads, issued before the weight loads and waited for before
// the first group's math), and the waves read them from there.  Loaded per
// group and wave they were a third of the kernel's memory instructions; the
// copy took the 27B-class batch-1 gate/up projection from 64.3 to 62.3 us
// and the O projection from 13.0 to 12.4 us, with bitwise-identical partial
// sums.  With 17-32 rows the activation fragments of a group (small,
// L2-resident) ride in the weight loads' register ring.
//
// Splitting K over the grid's z dimension gives enough waves to cover all 256
// CUs when a weight has few rows; each split writes float32 partial sums that
// the consumer kernel reduces in a fixed order (deterministic results).
//
// fp8 weights (e4m3fn + one float32 scale per output row) are widened to bf16
// when read from LDS (exact) and the scale is applied to the partial sums.
#include "common.h"
#include "dma_tile.h"
#include "kernels.h"

namespace dfl {

// One MFMA A-operand fragment (8 k-values of one row) read from the LDS copy
// of a weight group: bf16 16 bytes, fp8 8 bytes (widened), fp32 32 bytes.
template <typename TW> struct LdsFrag;
template <> struct LdsFrag<bf16_t> {
  typedef Frag8Bf16 frag;
  __device__ static void read(frag& f, const char* p) {
    f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  }
};
template <> struct LdsFrag<fp8_t> {
  typedef Frag8Bf16 frag;
  __device__ static void read(frag& f, const char* p) { fp8x8_to_frag(f, *reinterpret_cast<const u32x2*>(p)); }
};
template <> struct LdsFrag<float> {
  typedef Frag8F32 frag;
  __device__ static void read(frag& f, const char* p) { load_frag(f, reinterpret_cast<const float*>(p)); }
};

// XL: the activation operands come from an LDS copy of rows [m0, m0 + 16)
// (RM = 1, bf16 activations) over the K range [kb, ke): row q at xl + 2 q (ke - kb)
// (rows past the last one read the last); the caller has issued the global-to-
// LDS loads of that copy before run(), and run() waits for them after issuing
// its first weight loads, then meets the block's other waves at a barrier.
template <typename TA, typename TW, int RT, int RM, int NSG, bool XL = false>
struct GemmTile {
  typedef typename LdsFrag<TW>::frag WFr;
  typedef typename FragOf<TA>::type XFr;
  static constexpr int GB = 256;                   // bytes per row per group
  static constexpr int GK = GB / int(sizeof(TW));  // k per group
  static constexpr int STEPS = GK / 32;            // MFMA k-steps per group
  static constexpr int SB = 32 * int(sizeof(TW));  // bytes per row per k-step
  static constexpr int ROWB = GB + 16;             // LDS row stride
  static constexpr int NLD = 4 * RT;               // load instructions per group
  static constexpr int LDS_BYTES = 16 * RT * ROWB; // per wave
  static_assert(!XL || (RM == 1 && sizeof(TA) == 2), "LDS activations: 16 bf16 rows");

  // Accumulate rows [n0, n0 + 16 RT) x [m0, m0 + 16 RM) over k in [kb, ke)
  // (both multiples of 32).  `lds` is this wave's LDS_BYTES region.
  // Output: lane (r, g) holds acc[i][j][e] = y[row n0 + 16 i + 4 g + e][col m0 + 16 j + r].
  __device__ static void run(const TA* __restrict__ X, int64_t ldx, const TW* __restrict__ W,
                             int64_t ldw, int N, int Mact, int n0, int m0, int kb, int ke,
                             f32x4 (&acc)[RT][RM], char* lds, const char* xl = nullptr) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int r = lane & 15, g = lane >> 4;   // MFMA roles; for loads: g = row in 4, r = 16-byte piece
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < RM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (kb >= ke) return;
    const int ngroups = (ke - kb + GK - 1) / GK;
    const int kspan = ke - kb;
    // load side: instruction j reads row n0 + 4 j + g, bytes [16 r, 16 r + 16) of the group
    const char* wrow[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      int n = n0 + 4 * j + g;
      n = n < N ? n : N - 1;
      wrow[j] = reinterpret_cast<const char*>(W + int64_t(n) * ldw + kb) + 16 * r;
    }
    const TA* xrow[RM];
#pragma unroll
    for (int j = 0; j < RM; ++j) {
      int m = m0 + 16 * j + r;
      m = m < Mact ? m : Mact - 1;
      xrow[j] = X + int64_t(m) * ldx + kb + 8 * g;
    }
    u32x4 wr[NSG][NLD];
    XFr xr[NSG][STEPS][RM];
    auto load = [&](int s, int grp) {
      const int kg = grp * GK;
      // a 16-byte piece past the end of the K range is never multiplied; read
      // the group's first piece instead so the address stays inside the row
      const int off = (kg + (16 * (r + 1)) / int(sizeof(TW)) <= kspan ? kg * int(sizeof(TW)) : -16 * r);
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        wr[s][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[j] + off));
      if constexpr (!XL) {
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          const int kk = kg + 32 * st;
          const int kx = kk < kspan ? kk : 0;
#pragma unroll
          for (int j = 0; j < RM; ++j) load_frag(xr[s][st][j], xrow[j] + kx);
        }
      }
    };
    // LDS activation operand of lane (r, g): row min(r, rows - 1), k 8 g + ...
    const char* xlr = nullptr;
    if constexpr (XL) xlr = xl + (int64_t(min(r, min(16, Mact - m0) - 1)) * kspan + 8 * g) * 2;
    auto compute = [&](int s, int grp) {
#pragma unroll
      for (int j = 0; j < NLD; ++j)
        *reinterpret_cast<u32x4*>(lds + (4 * j + g) * ROWB + 16 * r) = wr[s][j];
      __builtin_amdgcn_wave_barrier();
      const int kg = grp * GK;
#pragma unroll
      for (int st = 0; st < STEPS; ++st) {
        if (kg + 32 * st < kspan) {
          XFr xf;
          if constexpr (XL) xf.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xlr + 2 * (kg + 32 * st)));
#pragma unroll
          for (int i = 0; i < RT; ++i) {
            WFr a;
            LdsFrag<TW>::read(a, lds + (16 * i + r) * ROWB + st * SB + g * (SB / 4));
#pragma unroll
            for (int j = 0; j < RM; ++j) acc[i][j] = mfma_k32(a, XL ? xf : xr[s][st][j], acc[i][j]);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    };
#pragma unroll
    for (int s = 0; s < NSG; ++s)
      if (s < ngroups) load(s, s);
    if constexpr (XL) {
      // the activation copy was requested before these weight loads
      if (ngroups >= NSG) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NSG * NLD));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      asm volatile("s_barrier" ::: "memory");
    }
    int base = 0;
    for (; base + 2 * NSG <= ngroups; base += NSG) {
#pragma unroll
      for (int s = 0; s < NSG; ++s) {
        compute(s, base + s);
        // keep the scheduler from hoisting later loads above this stage's
        // math (that would need a second copy of the register ring)
        __builtin_amdgcn_sched_barrier(0);
        load(s, base + NSG + s);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int s = 0; s < NSG; ++s) {
      if (base + s < ngroups) {
        compute(s, base + s);
        if (base + s + NSG < ngroups) load(s, base + s + NSG);
      }
    }
#pragma unroll
    for (int s = 0; s < NSG; ++s)
      if (base + NSG + s < ngroups) compute(s, base + NSG + s);
  }
};

// 1 / rms of an activation row from its per-column-block sums of squares
// (written by the residual/convolution kernel): the RMSNorm scale, applied
// to the GEMM result because it is one factor per row.
__device__ __forceinline__ float row_inv_rms(const RowScale& rs, int m) {
  if (!rs.sumsq) return 1.f;
  const float s = sum_in_order(rs.sumsq + int64_t(m) * rs.blocks, rs.blocks);
  return 1.0f / sqrtf(s * rs.inv_width + rs.eps);
}

// Largest activation copy: with the 34816 bytes of the waves' weight tiles,
// two blocks still fit a CU's 160 KiB of LDS.
constexpr int kGemmXlMaxBytes = 45056;

// Dynamic LDS bytes of the activation copy (XL): rows x k range in 16-byte
// pieces, whole rounds of 256 pieces (one per thread).
__host__ __device__ inline int gemm_xl_bytes(int rows, int kspan) {
  return (rows * (kspan / 8) + 255) / 256 * 4096;
}

// Partial-sum GEMM.  grid = (ceil(N / (64 RT)), ceil(M / (16 RM)), S); with
// XL, gemm_xl_bytes(min(16, M), k_split) bytes of dynamic LDS.
template <typename TA, typename TW, int RT, int RM, int NSG, bool XL = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void gemm_xwt_kernel(GemmArgs p) {
  typedef GemmTile<TA, TW, RT, RM, NSG, XL> Tile;
  __shared__ __attribute__((aligned(16))) char lds[4][Tile::LDS_BYTES];
  extern __shared__ __attribute__((aligned(16))) char xs[];
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int n0 = (blockIdx.x * 4 + wave) * 16 * RT;
  const int m0 = blockIdx.y * 16 * RM;
  if (m0 >= Mact) return;
  const int split = blockIdx.z % p.splits, group = blockIdx.z / p.splits;
  const void* Wp = p.groups > 1 ? p.Wg[group] : p.W;
  const float* scale = p.groups > 1 ? p.Sg[group] : p.scale;
  const int kb = split * p.k_split;
  const int ke = min(p.K, kb + p.k_split);
  const bool active = n0 < p.N && kb < ke;
  if constexpr (XL) {
    // every wave requests its share of the activation copy (block-uniform
    // trip count); lanes past the copy repeat its first piece into the
    // padding of the last round
    const int kspan = max(ke - kb, 0), cpr = kspan / 8;
    const int pieces = min(16, Mact - m0) * cpr;
    const bf16_t* X = static_cast<const bf16_t*>(p.X);
    for (int q = 0; q * 256 < pieces; ++q) {
      const int pc = q * 256 + int(threadIdx.x);
      const int row = pc < pieces ? pc / cpr : 0, c = pc < pieces ? pc - row * cpr : 0;
      lds_load16(X + int64_t(m0 + row) * p.ldx + kb + 8 * c, xs + 4096 * q + 1024 * wave);
    }
    if (!active) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      asm volatile("s_barrier" ::: "memory");   // the barrier of the waves that run the tile
      return;
    }
  } else {
    if (!active) return;
  }
  f32x4 acc[RT][RM];
  Tile::run(static_cast<const TA*>(p.X), p.ldx, static_cast<const TW*>(Wp), p.ldw, p.N, Mact, n0, m0,
            kb, ke, acc, lds[wave], xs);
  const int lane = threadIdx.x & (WAVE - 1);
  const int r = lane & 15, g = lane >> 4;
  float* P = p.P + int64_t(group) * p.group_stride + int64_t(split) * p.split_stride;
  float inv[RM];
#pragma unroll
  for (int j = 0; j < RM; ++j) inv[j] = row_inv_rms(p.rs, min(m0 + 16 * j + r, Mact - 1));
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int nb = n0 + 16 * i + 4 * g;
    float s[4] = {1.f, 1.f, 1.f, 1.f};
    if (scale) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = scale[min(nb + e, p.N - 1)];
    }
#pragma unroll
    for (int j = 0; j < RM; ++j) {
      const int m = m0 + 16 * j + r;
      if (m >= Mact) continue;
      float* dst = P + int64_t(m) * p.ldp + nb;
      f32x4 v = acc[i][j];
      v[0] *= s[0] * inv[j]; v[1] *= s[1] * inv[j]; v[2] *= s[2] * inv[j]; v[3] *= s[3] * inv[j];
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

// lm_head with the per-vocabulary-group top-k fused into the epilogue.
// grid = (ceil(V / kLmGroupIds), ceil(M / 16)); each block computes the
// logits of 128 vocabulary rows (32 per wave) for 16 activation rows over
// the full K, stages them in LDS, and keeps each activation row's k best
// (value desc, id asc) as 64-bit keys.  (256 rows per block in two passes
// of 32 rows per wave measured slower at the 27B workload: 292 against
// 272-278 us per step; each pass drained and refilled the load ring.)
template <typename TA, typename TW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void lmhead_topk_kernel(LmHeadArgs p) {
  constexpr int RT = 2;  // 32 rows per wave, 128 per block
  constexpr int G = kLmGroupIds;
  static_assert(G == 4 * 16 * RT, "one pass of 16 RT rows per wave");
  typedef GemmTile<TA, TW, RT, 1, 2> Tile;
  __shared__ __attribute__((aligned(16))) char lds[4][Tile::LDS_BYTES];
  __shared__ float logits[16][G + 4];
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m0 = blockIdx.y * 16;
  if (m0 >= Mact) return;
  const int wave = threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int r = lane & 15, g = lane >> 4;
  const int vbase = blockIdx.x * G;
  f32x4 acc[RT][1];
  const int n0 = vbase + wave * 16 * RT;
  if (n0 < p.N) {
    Tile::run(static_cast<const TA*>(p.X), p.ldx, static_cast<const TW*>(p.W), p.ldw, p.N, Mact, n0, m0, 0,
              p.K, acc, lds[wave]);
  } else {
#pragma unroll
    for (int i = 0; i < RT; ++i) acc[i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float inv = row_inv_rms(p.rs, min(m0 + r, Mact - 1));
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int nl = wave * 16 * RT + 16 * i + 4 * g;  // local vocab index
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int n = vbase + nl + e;
      float v = acc[i][0][e];
      if (p.scale) v *= p.scale[min(n, p.N - 1)];
      v *= inv;
      v = v + 0.0f;
      logits[r][nl + e] = v;
      const int m = m0 + r;
      if (p.debug_logits && n < p.N && m < Mact) p.debug_logits[int64_t(m) * p.N + n] = v;
    }
  }
  __syncthreads();
  // each wave ranks 4 of the 16 rows
  constexpr int KPL = G / WAVE;  // keys per lane
  for (int rr = 0; rr < 4; ++rr) {
    const int row = wave * 4 + rr;
    const int m = m0 + row;
    if (m >= Mact) break;
    uint64_t key[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      const int nl = lane + WAVE * e;
      const int n = vbase + nl;
      key[e] = n < p.N ? rank_key(logits[row][nl], uint32_t(n)) : 0ull;
    }
    // key t of this group at (m k + t) groups + group: the merge's lanes
    // then read consecutive groups with coalesced loads
    uint64_t* out = p.cand + int64_t(m) * p.k * p.groups + blockIdx.x;
    for (int t = 0; t < p.k; ++t) {
      uint64_t best = key[0];
#pragma unroll
      for (int e = 1; e < KPL; ++e) best = key[e] > best ? key[e] : best;
      best = wave_max_u64(best);
#pragma unroll
      for (int e = 0; e < KPL; ++e)
        if (key[e] == best) key[e] = 0ull;
      if (lane == 0) out[int64_t(t) * p.groups] = best;
    }
  }
}

// First fold of many candidate lists (k <= 16): block (c, m), one wave, merges
// lists [64 c, 64 c + 64) of row m -- one list per lane, then six xor rounds
// of the two-list merge below -- into the 16 largest keys, written sorted at
// out[(m nc + c) 16] (zeros where fewer).  The rows' nc lists then go to the
// final merge: a row's lists are folded by 64 x the rows' blocks at once
// instead of by the 256 threads of one block.
__global__ __launch_bounds__(64) void topk_premerge_kernel(TopkMergeArgs p, uint64_t* out, int nc) {
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m = blockIdx.y;
  if (m >= Mact) return;
  const int lane = threadIdx.x;
  const uint64_t* c = p.cand + int64_t(m) * p.count;
  const int groups = p.count / p.glen;
  const int gi = blockIdx.x * WAVE + lane;
  uint64_t best[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    best[j] = (gi < groups && j < p.glen) ? c[int64_t(gi) * p.lstride + int64_t(j) * p.kstride] : 0ull;
  for (int d = 1; d < WAVE; d <<= 1) {
    uint64_t brev[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) brev[j] = __shfl_xor(best[15 - j], d, WAVE);
    bitonic_top<16>(best, brev);
  }
  if (lane < 16) {
    uint64_t v = best[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) v = lane == j ? best[j] : v;
    out[(int64_t(m) * nc + blockIdx.x) * 16 + lane] = v;
  }
}

// Final top-k over the per-group candidates of one row, then the logit
// transform.  grid = (M), block = 256.  The lm_head kernels emit sorted
// lists of glen keys (largest first; glen <= KMAX) and keys are distinct
// (ids are).  Each thread folds whole groups into a sorted list of KMAX keys;
// two sorted lists combine into the KMAX largest of their union by taking
// max(a[i], b[KMAX-1-i]) (a bitonic sequence) and sorting that with a
// bitonic half-cleaner cascade.  Lists are combined across lanes by xor
// shuffles, then across the block's waves through LDS.  k <= KMAX.
template <int KMAX, int NT>
__global__ __launch_bounds__(NT) void topk_merge_kernel(TopkMergeArgs p) {
  constexpr int NW = NT / WAVE;
  __shared__ uint64_t lists[NW * KMAX];
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m = blockIdx.x;
  if (m >= Mact) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1), wave = tid / WAVE;
  const uint64_t* c = p.cand + int64_t(m) * p.count;
  const int groups = p.count / p.glen;
  uint64_t best[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) best[j] = 0ull;
  // each thread's next list is loaded while the current one is merged
  auto load_rev = [&](uint64_t (&dst)[KMAX], int gi) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int src = KMAX - 1 - j;                 // reversed: ascending
      dst[j] = (gi < groups && src < p.glen) ? c[int64_t(gi) * p.lstride + int64_t(src) * p.kstride] : 0ull;
    }
  };
  uint64_t nxt[KMAX];
  load_rev(nxt, tid);
  for (int gi = tid; gi < groups; gi += NT) {
    uint64_t brev[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) brev[j] = nxt[j];
    load_rev(nxt, gi + NT);
    bitonic_top<KMAX>(best, brev);
  }
  for (int d = 1; d < WAVE; d <<= 1) {
    uint64_t brev[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) brev[j] = __shfl_xor(best[KMAX - 1 - j], d, WAVE);
    bitonic_top<KMAX>(best, brev);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) lists[wave * KMAX + j] = best[j];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) best[j] = lane < NW ? lists[lane * KMAX + j] : 0ull;
    for (int d = 1; d < NW; d <<= 1) {
      uint64_t brev[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) brev[j] = __shfl_xor(best[KMAX - 1 - j], d, WAVE);
      bitonic_top<KMAX>(best, brev);
    }
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < KMAX; ++t) {
        if (t < p.k) {
          float z = p.multiplier * key_val(best[t]);
          if (p.softcap > 0.f) z = p.softcap * tanhf(z / p.softcap);
          p.ids[int64_t(m) * p.k + t] = int32_t(key_id(best[t]));
          p.vals[int64_t(m) * p.k + t] = z;
        }
      }
    }
  }
}

// The same result for k > 16: k rounds, each taking the largest key below the
// previous one with a block-wide maximum over all candidates.
__global__ __launch_bounds__(256) void topk_merge_rounds_kernel(TopkMergeArgs p) {
  __shared__ uint64_t red[4];
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m = blockIdx.x;
  if (m >= Mact) return;
  const uint64_t* c = p.cand + int64_t(m) * p.count;
  uint64_t prev = ~0ull;
  for (int t = 0; t < p.k; ++t) {
    uint64_t best = 0ull;
#pragma unroll 8
    for (int i = threadIdx.x; i < p.count; i += blockDim.x) {
      const uint64_t v = c[i];
      best = (v < prev && v > best) ? v : best;
    }
    best = wave_max_u64(best);
    if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = best;
    __syncthreads();
    best = red[0];
    for (int w = 1; w < int(blockDim.x / WAVE); ++w) best = red[w] > best ? red[w] : best;
    __syncthreads();
    prev = best;
    if (threadIdx.x == 0) {
      float z = p.multiplier * key_val(best);
      if (p.softcap > 0.f) z = p.softcap * tanhf(z / p.softcap);
      p.ids[int64_t(m) * p.k + t] = int32_t(key_id(best));
      p.vals[int64_t(m) * p.k + t] = z;
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <typename TA, typename TW, int RT, int RM, int NSG, bool XL = false>
static void launch_gemm_t(const GemmArgs& a, hipStream_t s) {
  dim3 grid((a.N + 64 * RT - 1) / (64 * RT), (a.M + 16 * RM - 1) / (16 * RM), a.splits * max(1, a.groups));
  const unsigned xbytes = XL ? unsigned(gemm_xl_bytes(min(16, a.M), a.k_split)) : 0u;
  hipLaunchKernelGGL((gemm_xwt_kernel<TA, TW, RT, RM, NSG, XL>), grid, dim3(256), xbytes, s, a);
}

// 32 weight rows per wave (128 per block); two groups in flight for up to 16
// activation rows, one when a group carries more activation fragments.
template <typename TA, typename TW>
static void launch_gemm_rm(const GemmArgs& a, hipStream_t s) {
  constexpr int NSG1 = sizeof(TW) == 1 ? 1 : 2;  // fp8 groups carry twice the activation fragments
  if constexpr (sizeof(TA) == 2) {
    // activations through LDS while the copy leaves two blocks per CU
    if (a.M <= 16 && gemm_xl_bytes(a.M, a.k_split) <= kGemmXlMaxBytes) {
      launch_gemm_t<TA, TW, 2, 1, 2, true>(a, s);
      return;
    }
  }
  if (a.M <= 16) launch_gemm_t<TA, TW, 2, 1, NSG1>(a, s);
  else if (a.M <= 32) launch_gemm_t<TA, TW, 2, 2, 1>(a, s);
  else launch_gemm_t<TA, TW, 2, 4, 1>(a, s);
}

int gemm_rows_per_block(int weight_dtype, int M) {
  (void)weight_dtype;
  (void)M;
  return 128;
}

bool tiled_epi_fusable(const GemmArgs& a);

bool gemm_epi_fusable(int weight_dtype, const GemmArgs& a) {
  return weight_dtype != 0 && gemm_tiled_ok(weight_dtype, a.M, a.K) && tiled_epi_fusable(a);
}

void launch_gemm(int weight_dtype, const GemmArgs& a, hipStream_t s) {
  if (gemm_tiled_ok(weight_dtype, a.M, a.K)) {
    launch_gemm_tiled(weight_dtype, a, s);
    return;
  }
  switch (weight_dtype) {
    case 0: launch_gemm_rm<float, float>(a, s); break;
    case 1: launch_gemm_rm<bf16_t, bf16_t>(a, s); break;
    default: launch_gemm_rm<bf16_t, fp8_t>(a, s); break;
  }
}

void launch_lmhead_topk(int weight_dtype, const LmHeadArgs& a, hipStream_t s) {
  if (lmhead_tiled_ok(weight_dtype, a.M, a.K, a.k)) {
    launch_lmhead_tiled(weight_dtype, a, s);
    return;
  }
  dim3 grid(a.groups, (a.M + 15) / 16);
  switch (weight_dtype) {
    case 0: hipLaunchKernelGGL((lmhead_topk_kernel<float, float>), grid, dim3(256), 0, s, a); break;
    case 1: hipLaunchKernelGGL((lmhead_topk_kernel<bf16_t, bf16_t>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((lmhead_topk_kernel<bf16_t, fp8_t>), grid, dim3(256), 0, s, a); break;
  }
}

void launch_topk_merge(const TopkMergeArgs& a, hipStream_t s) {
  // (1024 threads per row, one list each, measured slower: 22 vs 19 us at
  // 7 rows, 124 vs 73 us at 1792 rows -- the shuffle rounds dominate)
  if (a.k <= 16 && a.count / a.glen <= 64)
    hipLaunchKernelGGL((topk_merge_kernel<16, 64>), dim3(a.M), dim3(64), 0, s, a);
  else if (a.k <= 16)
    hipLaunchKernelGGL((topk_merge_kernel<16, 256>), dim3(a.M), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(topk_merge_rounds_kernel, dim3(a.M), dim3(256), 0, s, a);
}

int topk_premerge_lists(int lists) { return (lists + WAVE - 1) / WAVE; }

void launch_topk_premerge(const TopkMergeArgs& a, uint64_t* out, hipStream_t s) {
  const int nc = topk_premerge_lists(a.count / a.glen);
  hipLaunchKernelGGL(topk_premerge_kernel, dim3(nc, a.M), dim3(64), 0, s, a, out, nc);
}

}  // namespace dfl

// Non-causal block attention over context + block keys (NeMo AutoModel page,
// "What is DFlash?": every block slot sees the whole context and every other
// slot; no mask), grouped KV heads.
//
// Work split ("flash-decoding"): the keys of one (sequence, kv head) are cut
// into chunks of chunk_keys (a multiple of the KT-key sub-chunk).  A block of
// four waves owns one chunk and up to 64 query slots (slot s = t * group + j
// for block row t and q head j of the group); wave w owns query tile w (16
// slots).  Per sub-chunk the block stages K [KT][d] and V^T [d][KT] in LDS
// with coalesced 16-byte loads (V zeroed outside the valid key range); the
// global loads of the next sub-chunk are issued into registers right after
// the LDS hand-off, so they are in flight while the waves compute.  Each
// wave then computes S^T = K Q^T on the matrix cores (keys as rows) per
// 32-key tile, runs an online softmax per query in registers and accumulates
// O^T = V^T P^T, so the probabilities are already laid out as the second MFMA
// operand.  Each wave writes one (max, sum, O) partial per query; a second
// kernel merges the chunks (log-sum-exp, fixed order).  When one chunk holds
// every key (large batches) the wave normalises and writes the output itself
// and the merge is not launched; the result is the same bits the merge would
// give (its weight is exp2(0) = 1 and its sum the chunk's own).
//
// Cache layouts (per layer): K [Bcap][nkv][Lmax][d] (rows of d), V
// [Bcap][nkv][d][Lmax] (position fastest), so both staging loads are
// contiguous.
#include "common.h"
#include "kernels.h"

namespace dfl {

template <typename T> struct AttnFrag;
template <> struct AttnFrag<bf16_t> {
  typedef Frag8Bf16 frag;
  __device__ static void from_f32(frag& f, const float (&p)[8]) {
    u32x4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = f32x2_to_bf16x2(p[2 * j], p[2 * j + 1]);
    f.v = __builtin_bit_cast(bf16x8, u);
  }
};
template <> struct AttnFrag<float> {
  typedef Frag8F32 frag;
  __device__ static void from_f32(frag& f, const float (&p)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = p[j];
  }
};

__device__ __forceinline__ float exp2_safe(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes of T (8 bf16 or 4 floats) with the elements whose key is outside
// [lo, hi) set to zero; key0 is the key of the first element.
template <typename T> struct Piece;
template <> struct Piece<bf16_t> {
  static constexpr int N = 8;
  __device__ static u32x4 masked(u32x4 u, int key0, int lo, int hi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = key0 + 2 * j;
      const uint32_t m0 = (k >= lo && k < hi) ? 0x0000FFFFu : 0u;
      const uint32_t m1 = (k + 1 >= lo && k + 1 < hi) ? 0xFFFF0000u : 0u;
      u[j] &= (m0 | m1);
    }
    return u;
  }
};
template <> struct Piece<float> {
  static constexpr int N = 4;
  __device__ static u32x4 masked(u32x4 u, int key0, int lo, int hi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = (key0 + j >= lo && key0 + j < hi) ? u[j] : 0u;
    return u;
  }
};

// 64-key sub-chunks keep the LDS of a block at ~36 KB (bf16, d 128), so
// three blocks share a CU; with the loads of the next sub-chunk in flight
// during the MFMAs this measured 3.7 -> 5.0 TB/s on 8192-key contexts
// (128-key sub-chunks without the overlap: two blocks per CU).
template <typename T, int D>
struct AttnShape {
  static constexpr int KT = 64;                 // keys per LDS sub-chunk
  static constexpr int PAD = 16 / sizeof(T);    // 16 bytes of row padding
  static constexpr int OCC = (sizeof(T) == 2 && D <= 128) ? 3 : 1;  // blocks per CU asked of the compiler
};

template <typename T, int D>
__global__ __launch_bounds__(256, (AttnShape<T, D>::OCC)) void attn_partial_kernel(AttnArgs p) {
  typedef typename AttnFrag<T>::frag Frag;
  constexpr int KT = AttnShape<T, D>::KT;
  constexpr int PAD = AttnShape<T, D>::PAD;
  constexpr int DS = (D + 31) / 32;  // QK^T contraction steps
  constexpr int DT = D / 16;         // output d tiles
  constexpr int PN = Piece<T>::N;    // elements per 16-byte piece
  __shared__ __attribute__((aligned(16))) T Ks[KT][D + PAD];
  __shared__ __attribute__((aligned(16))) T Vs[D][KT + PAD];

  const int c = blockIdx.x;
  const int g = blockIdx.y % p.nkv, qg = blockIdx.y / p.nkv;
  const int b = blockIdx.z;
  const int grp = p.nq / p.nkv, QS = p.bs * grp;
  const int L = p.ctx_lens[b];
  const int n_end = min(L + p.bs, p.Lmax);
  const int lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int lo_al = lo & ~31;
  const int cstart = lo_al + c * p.chunk_keys;
  const int cend = min(cstart + p.chunk_keys, n_end);

  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid & (WAVE - 1);
  const int r = lane & 15, gq = lane >> 4;
  const int slot0 = qg * 64 + wave * 16;  // first query slot of this wave
  const bool active = slot0 < QS;
  // single-chunk mode: lane (r, gq) writes dims 16 dt + 4 gq .. + 3 of slot r
  auto write_out = [&](const f32x4* acc, float inv) {
    const int s = slot0 + r;
    if (!active || s >= QS) return;
    T* out = static_cast<T*>(p.o);
    const int64_t ob = (int64_t(b * p.bs + s / grp) * p.nq + g * grp + s % grp) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) Act<T>::store(out, ob + dt * 16 + 4 * gq + e, acc[dt][e] * inv);
  };
  if (cstart >= n_end || L < 0) {
    if (p.nchunks == 1) {  // no keys: the merge would write zeros
      f32x4 z[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) z[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      write_out(z, 0.f);
    }
    return;
  }

  // this wave's queries, straight into registers (zeros past the last slot)
  Frag qf[DS];
  {
    const int s = slot0 + r;
    const T* Q = static_cast<const T*>(p.q);
    const int t = s / grp, h = g * grp + s % grp;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      const int d0 = 32 * st + 8 * gq;
      if (active && s < QS && d0 < D) load_frag(qf[st], Q + (int64_t(b * p.bs + t) * p.nq + h) * D + d0);
      else zero_frag(qf[st]);
    }
  }

  const T* Kb = static_cast<const T*>(p.k_layer) + (int64_t(b) * p.nkv + g) * p.Lmax * D;
  const T* Vb = static_cast<const T*>(p.v_layer) + (int64_t(b) * p.nkv + g) * D * int64_t(p.Lmax);

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- K rows [ks, ks + KT) and V^T columns [ks, ks + KT) into registers ---
  constexpr int KP = KT * D / PN;  // 16-byte pieces of K (and of V)
  constexpr int NP = (KP + 255) / 256;
  u32x4 kv[NP], vv[NP];
  auto fetch = [&](int ks) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = u * 256 + tid;
      const int row = i / (D / PN), col = (i % (D / PN)) * PN;
      const int key = min(ks + row, p.Lmax - 1);
      kv[u] = i < KP ? *reinterpret_cast<const u32x4*>(Kb + int64_t(key) * D + col) : u32x4{0u, 0u, 0u, 0u};
      const int dd = i / (KT / PN), kc = (i % (KT / PN)) * PN;
      const int key0 = min(ks + kc, p.Lmax - PN);
      vv[u] = i < KP ? *reinterpret_cast<const u32x4*>(Vb + int64_t(dd) * p.Lmax + key0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  fetch(cstart);
  for (int ks = cstart; ks < cend; ks += KT) {
    // ---- registers -> LDS, then start the next sub-chunk's loads ----------
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = u * 256 + tid;
      if (i < KP) {
        const int row = i / (D / PN), col = (i % (D / PN)) * PN;
        *reinterpret_cast<u32x4*>(&Ks[row][col]) = kv[u];
        const int dd = i / (KT / PN), kc = (i % (KT / PN)) * PN;
        *reinterpret_cast<u32x4*>(&Vs[dd][kc]) = Piece<T>::masked(vv[u], ks + kc, lo, n_end);
      }
    }
    __syncthreads();
    if (ks + KT < cend) fetch(ks + KT);
    if (active) {
#pragma unroll 1
      for (int kt = 0; kt < KT; kt += 32) {
        const int k0 = ks + kt;
        if (k0 >= cend) break;
        // K rows: MFMA "a" row rho <-> key 8*(rho/4) + rho%4, "b" <-> that + 4, so
        // lane (r, g) ends up holding keys k0 + 8g .. k0 + 8g + 7 of its query.
        const int ra = kt + 8 * (r >> 2) + (r & 3);
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < DS; ++st) {
          const int d0 = 32 * st + 8 * gq;
          Frag ka, kb;
          if (d0 < D) {
            load_frag(ka, &Ks[ra][d0]);
            load_frag(kb, &Ks[ra + 4][d0]);
          } else {
            zero_frag(ka);
            zero_frag(kb);
          }
          sa = mfma_k32(ka, qf[st], sa);
          sb = mfma_k32(kb, qf[st], sb);
        }
        const int kk0 = k0 + 8 * gq;
        float sc[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ka_ = kk0 + e, kb_ = kk0 + 4 + e;
          sc[e] = (ka_ >= lo && ka_ < n_end) ? sa[e] * p.scale_log2 : -INFINITY;
          sc[4 + e] = (kb_ >= lo && kb_ < n_end) ? sb[e] * p.scale_log2 : -INFINITY;
        }
        float tmax = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, WAVE));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, WAVE));
        const float mnew = fmaxf(m_run, tmax);
        float pr[8];
        float alpha = 1.f, psum = 0.f;
        if (mnew == -INFINITY) {
#pragma unroll
          for (int j = 0; j < 8; ++j) pr[j] = 0.f;
        } else {
          alpha = exp2_safe(m_run - mnew);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pr[j] = exp2_safe(sc[j] - mnew);
            psum += pr[j];
          }
        }
        m_run = mnew;
        l_run = l_run * alpha + psum;
        Frag pf;
        AttnFrag<T>::from_f32(pf, pr);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          Frag vf;
          load_frag(vf, &Vs[dt * 16 + r][kt + 8 * gq]);
          o[dt] *= alpha;
          o[dt] = mfma_k32(vf, pf, o[dt]);
        }
      }
    }
    __syncthreads();
  }
  if (!active) return;
  // each lane holds a partial sum over its keys: total per query
  l_run += __shfl_xor(l_run, 16, WAVE);
  l_run += __shfl_xor(l_run, 32, WAVE);
  if (p.nchunks == 1) {
    write_out(o, l_run > 0.f ? 1.f / l_run : 0.f);
    return;
  }
  const int s = slot0 + r;
  if (s >= QS) return;
  const int64_t prow = ((int64_t(b) * p.nkv + g) * p.nchunks + c) * QS + s;
  float* po = p.part_o + prow * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(po + dt * 16 + 4 * gq) = o[dt];
  if (gq == 0) {
    p.part_ml[prow * 2 + 0] = m_run;
    p.part_ml[prow * 2 + 1] = l_run;
  }
}

// One wave per (sequence, block row, q head): merge the chunk partials.
// Lanes read the chunks' (max, sum) in parallel.  For the output, lane
// (cs, q) owns the 4 dimensions [4q, 4q + 4) and the chunks c = cs, cs + CS,
// ... (CS = 64 / (d / 4) chunk subsets); the subsets are then added with
// shuffles in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnCombineArgs p) {
  const int idx = blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  if (idx >= p.B * p.bs * p.nq) return;
  const int h = idx % p.nq, t = (idx / p.nq) % p.bs, b = idx / (p.nq * p.bs);
  const int grp = p.nq / p.nkv, g = h / grp, QS = p.bs * grp;
  const int s = t * grp + h % grp;
  const int L = p.ctx_lens[b];
  const int n_end = min(L + p.bs, p.Lmax);
  const int lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int lo_al = lo & ~31;
  const int CH = p.chunk_keys;
  const int nvalid = (L < 0 || n_end <= lo_al) ? 0 : min(p.nchunks, (n_end - lo_al + CH - 1) / CH);
  const int64_t cbase = (int64_t(b) * p.nkv + g) * p.nchunks;
  const f32x2* ml = reinterpret_cast<const f32x2*>(p.part_ml);
  // up to 64 chunks: lane l reads chunk l's (max, sum) once and keeps it;
  // more chunks: two passes (max, then the rescaled sums)
  const bool one_pass = nvalid <= WAVE;
  const f32x2 first = (one_pass && lane < nvalid) ? ml[(cbase + lane) * QS + s] : f32x2{-INFINITY, 0.f};
  float M, lsum;
  if (one_pass) {
    M = wave_max(first[0]);
    lsum = wave_sum(first[0] != -INFINITY ? first[1] * exp2_safe(first[0] - M) : 0.f);
  } else {
    float m = -INFINITY;
    for (int c = lane; c < nvalid; c += WAVE) m = fmaxf(m, ml[(cbase + c) * QS + s][0]);
    M = wave_max(m);
    float l = 0.f;
    for (int c = lane; c < nvalid; c += WAVE) {
      const f32x2 v = ml[(cbase + c) * QS + s];
      if (v[0] != -INFINITY) l += v[1] * exp2_safe(v[0] - M);
    }
    lsum = wave_sum(l);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;

  const int nq4 = p.d / 4;                  // 4 .. 64
  const int CS = WAVE / nq4;                // chunk subsets
  const int q = lane % nq4, cs = lane / nq4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int cb = 0; cb < nvalid; cb += WAVE) {
    float mc = first[0];
    if (!one_pass) mc = cb + lane < nvalid ? ml[(cbase + cb + lane) * QS + s][0] : -INFINITY;
    const float wgt = mc != -INFINITY ? exp2_safe(mc - M) : 0.f;
    const int n = min(WAVE, nvalid - cb);
    for (int c0 = 0; c0 < n; c0 += 4 * CS) {  // same trip count on every lane
      f32x4 v[4];
      float w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int c = c0 + cs + u * CS;
        const bool ok = c < n;
        v[u] = *reinterpret_cast<const f32x4*>(p.part_o + ((cbase + cb + (ok ? c : 0)) * QS + s) * p.d + 4 * q);
        const float wsrc = __shfl(wgt, ok ? c : 0, WAVE);
        w[u] = ok ? wsrc : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += v[u] * w[u];
    }
  }
  for (int off = nq4; off < WAVE; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off, WAVE);
  }
  if (cs == 0) {
    T* out = static_cast<T*>(p.o);
    const int64_t o = (int64_t(b * p.bs + t) * p.nq + h) * p.d + 4 * q;
#pragma unroll
    for (int e = 0; e < 4; ++e) Act<T>::store(out, o + e, acc[e] * inv);
  }
}

bool attn_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

int attn_sub_chunk(bool f32, int d) {
  return f32 ? AttnShape<float, 16>::KT : (d == 256 ? AttnShape<bf16_t, 256>::KT : AttnShape<bf16_t, 128>::KT);
}

template <typename T>
static void launch_attn_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.nchunks, a.nkv * a.qgroups, a.B);
  switch (a.d) {
    case 16: hipLaunchKernelGGL((attn_partial_kernel<T, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((attn_partial_kernel<T, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((attn_partial_kernel<T, 64>), grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((attn_partial_kernel<T, 128>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_partial_kernel<T, 256>), grid, dim3(256), 0, s, a); break;
  }
}

void launch_attention(bool f32, const AttnArgs& a, hipStream_t s) {
  if (f32) launch_attn_t<float>(a, s);
  else launch_attn_t<bf16_t>(a, s);
}

void launch_attn_combine(bool f32, const AttnCombineArgs& a, hipStream_t s) {
  dim3 grid((a.B * a.bs * a.nq + 3) / 4);
  if (f32) hipLaunchKernelGGL(attn_combine_kernel<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, grid, dim3(256), 0, s, a);
}

}  // namespace dfl

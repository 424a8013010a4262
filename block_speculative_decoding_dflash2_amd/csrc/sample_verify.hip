// Sampled (rejection) verification of a deterministic draft path.
//
// NeMo AutoModel page, "Key Config Fields" (paragraph on spec_generate):
// temperature, top-p and top-k truncate the target's distribution, and the
// drafts are verified against that distribution by rejection sampling, so
// sampled decoding keeps the target's own output distribution.  The DFlash2
// path comes from the selector lattice (llama-cpp-python wiki, "Configuration
// Notes"), so the draft distribution is a point mass on each chosen token and
// speculative sampling reduces to: accept d_i when u_i < p_i(d_i); at the
// first rejection draw from p_i with d_i struck out; when every proposed
// draft is accepted draw from the next row.
//
// Per row (one workgroup of 1024 threads per target row), the truncated
// distribution is p_v = e_v / S over the kept set {v : key_v >= theta}, with
// e_v = exp((z_v - m) / T).  theta and S are found without sorting the
// vocabulary:
//   * top-k, common case: the row's first ids estimate (from a histogram of
//     their keys) a bin low enough that at least k elements lie at or above
//     it; one pass takes the row maximum and collects every element at or
//     above that bin into an LDS list, which is sorted exactly;
//   * top-k, otherwise (too few or too many collected): the k-th largest
//     value by a radix select over the order-preserving 32-bit key of each
//     logit (11 + 11 + 10 bit digits, one histogram pass per digit, LDS
//     histograms), switching to the sorted list as soon as every element at
//     or above the current bin fits it (<= 2048 entries);
//   * top-p: the same radix select on the kept mass instead of the count,
//     or the sorted list when it holds the kept set.
// Weights are accumulated as 64-bit fixed-point integers E_v =
// round(e_v * 2^s), s = 52 - ceil(log2 V), so every sum (histogram bins,
// prefixes, totals) is exact and independent of the order of the atomics:
// the sums of the sub-bins of a bin equal the bin, results are run-to-run
// deterministic, and every total is exact in a double.  The decisions
// u_i * S < E_d and the inverse-CDF draw are taken on these integers.
// A second kernel (one workgroup per sequence) walks the accept decisions and
// draws the bonus token: from the kept set the row pass handed over when it
// is small, else by an exact prefix scan over the stop row.
#include <cfloat>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace dfl {

namespace {

constexpr int SV_THREADS = 1024;
constexpr int SV_WAVES = SV_THREADS / WAVE;
constexpr int SV_BINS = 2048;
constexpr int SV_CAP = 2048;  // LDS list capacity; two entries per thread

// NaN -> -inf (probability 0), +inf -> the largest float, -0.0 -> +0.0.
__device__ __forceinline__ float sv_clean(float z) {
  z = z + 0.0f;
  if (z != z) return -INFINITY;
  return fminf(z, FLT_MAX);
}
// Order-preserving key of a cleaned value.
__device__ __forceinline__ uint32_t sv_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float sv_val(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

struct SvWeight {
  uint32_t mkey;
  float m, temp, qscale;
  // Fixed-point weight of the value with key k: the row maximum weighs
  // exactly 2^s (also when the maximum is -inf).
  __device__ __forceinline__ uint64_t operator()(uint32_t k) const {
    const float e = k == mkey ? 1.0f : expf((sv_val(k) - m) / temp);
    return __float2ull_rn(e * qscale);
  }
};

// Radix digits: level 0 = key bits 31..21, level 1 = 20..10, level 2 = 9..0.
__device__ __forceinline__ int sv_shift(int level) { return level == 0 ? 21 : (level == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t sv_digit(uint32_t k, int level) {
  return level == 0 ? (k >> 21) : (level == 1 ? ((k >> 10) & 2047u) : (k & 1023u));
}
// Does key k lie in the bin chosen so far (prefix = the digits above level)?
__device__ __forceinline__ bool sv_in_prefix(uint32_t k, int level, uint32_t prefix) {
  return level == 0 || (k >> (level == 1 ? 21 : 10)) == prefix;
}

struct SvShared {
  uint32_t cnt[SV_BINS];
  uint64_t mass[SV_BINS];
  uint64_t list[SV_CAP];   // (key << 32) | (~id): sorted descending = value desc, id asc
  uint64_t pre[SV_CAP];    // weights, then their exclusive prefix sums
  uint64_t scan[2 * SV_WAVES];
  uint32_t red[SV_WAVES];
  uint32_t nlist;
  uint32_t fbin;
  uint64_t fabove_w, fabove_c, fbin_w, fbin_c, total_w;
};

// Exclusive prefix sums of two u64 values over the block (thread order);
// totals of both are returned through tot_a / tot_b.
__device__ __forceinline__ void sv_scan2(uint64_t& a, uint64_t& b, uint64_t& tot_a, uint64_t& tot_b,
                                         uint64_t* sh) {
  const int lane = threadIdx.x & (WAVE - 1), wave = threadIdx.x / WAVE;
  uint64_t ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const uint64_t ta = __shfl_up(ia, o, WAVE), tb = __shfl_up(ib, o, WAVE);
    if (lane >= o) { ia += ta; ib += tb; }
  }
  if (lane == WAVE - 1) { sh[wave] = ia; sh[SV_WAVES + wave] = ib; }
  __syncthreads();
  uint64_t pa = 0, pb = 0, sa = 0, sb = 0;
  for (int w = 0; w < SV_WAVES; ++w) {
    const uint64_t xa = sh[w], xb = sh[SV_WAVES + w];
    if (w < wave) { pa += xa; pb += xb; }
    sa += xa; sb += xb;
  }
  a = pa + ia - a;
  b = pb + ib - b;
  tot_a = sa; tot_b = sb;
  __syncthreads();
}

// Bins are ranked from the top (bin nb-1 first).  Finds the bin b with
// base + above(b) < X <= base + above(b) + h(b), h = mass (by_mass) or count,
// above(b) = the sum of h over the bins above b.  Exactly one bin satisfies
// it when base < X <= base + sum(h), since the sums are exact integers.
__device__ void sv_find(SvShared& sh, int nb, bool by_mass, double X, uint64_t base) {
  const int t = threadIdx.x;
  const int bhi = nb - 1 - 2 * t, blo = bhi - 1;
  uint64_t whi = 0, wlo = 0, chi = 0, clo = 0;
  if (bhi >= 0) { chi = sh.cnt[bhi]; whi = by_mass ? sh.mass[bhi] : chi; }
  if (blo >= 0) { clo = sh.cnt[blo]; wlo = by_mass ? sh.mass[blo] : clo; }
  uint64_t ew = whi + wlo, ec = chi + clo, tw, tc;
  sv_scan2(ew, ec, tw, tc, sh.scan);
  if (t == 0) sh.total_w = tw;
  if (bhi >= 0 && double(base + ew) < X && X <= double(base + ew + whi)) {
    sh.fbin = uint32_t(bhi); sh.fabove_w = ew; sh.fabove_c = ec; sh.fbin_w = whi; sh.fbin_c = chi;
  }
  if (blo >= 0 && double(base + ew + whi) < X && X <= double(base + ew + whi + wlo)) {
    sh.fbin = uint32_t(blo); sh.fabove_w = ew + whi; sh.fabove_c = ec + chi; sh.fbin_w = wlo; sh.fbin_c = clo;
  }
  __syncthreads();
}

// Calls f(id, value) for every element of the row, eight 16-byte loads in
// flight per thread (a row is read by one block, so the loads in flight set
// its rate).
template <class F>
__device__ __forceinline__ void sv_for_row(const float* __restrict__ z, int V, bool vec, F&& f) {
  if (vec) {
    const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
    const int n4 = V >> 2;
    for (int i0 = threadIdx.x; i0 < n4; i0 += 8 * SV_THREADS) {
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * SV_THREADS;
        x[u] = i < n4 ? __builtin_nontemporal_load(z4 + i) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * SV_THREADS;
        if (i < n4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) f(4 * i + e, x[u][e]);
        }
      }
    }
  } else {
    for (int i = threadIdx.x; i < V; i += SV_THREADS) f(i, z[i]);
  }
}

__device__ __forceinline__ void sv_clear(SvShared& sh, bool mass) {
  for (int i = threadIdx.x; i < SV_BINS; i += SV_THREADS) {
    sh.cnt[i] = 0u;
    if (mass) sh.mass[i] = 0ull;
  }
  __syncthreads();
}

// Histogram (count, and mass when w != nullptr) of digit `level` over the
// keys >= floor_key inside the bin `prefix`.
__device__ void sv_hist(SvShared& sh, const float* z, int V, bool vec, int level, uint32_t prefix,
                        uint32_t floor_key, const SvWeight* w) {
  sv_clear(sh, w != nullptr);
  sv_for_row(z, V, vec, [&](int, float x) {
    const uint32_t k = sv_key(sv_clean(x));
    if (k >= floor_key && sv_in_prefix(k, level, prefix)) {
      const uint32_t d = sv_digit(k, level);
      atomicAdd(&sh.cnt[d], 1u);
      if (w) atomicAdd(reinterpret_cast<unsigned long long*>(&sh.mass[d]), (unsigned long long)(*w)(k));
    }
  });
  __syncthreads();
}

// Collects every element with key >= lo into the list (entries past the
// capacity are counted, not stored); returns the count.
__device__ uint32_t sv_collect(SvShared& sh, const float* z, int V, bool vec, uint32_t lo) {
  if (threadIdx.x == 0) sh.nlist = 0u;
  __syncthreads();
  sv_for_row(z, V, vec, [&](int id, float x) {
    const uint32_t k = sv_key(sv_clean(x));
    if (k >= lo) {
      const uint32_t slot = atomicAdd(&sh.nlist, 1u);
      if (slot < uint32_t(SV_CAP)) sh.list[slot] = (uint64_t(k) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(id));
    }
  });
  __syncthreads();
  const uint32_t n = sh.nlist;
  __syncthreads();
  return n;
}

// Sorts the first n (<= capacity) list entries descending (value desc, id asc).
__device__ void sv_sort(SvShared& sh, int n) {
  int N = 2;
  while (N < n) N <<= 1;
  for (int i = n + threadIdx.x; i < N; i += SV_THREADS) sh.list[i] = 0ull;
  __syncthreads();
  // bitonic sort, descending; N / 2 <= SV_THREADS compare-exchanges per stage
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int t = threadIdx.x;
      if (t < N / 2) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t a = sh.list[i], b = sh.list[j];
        if ((a < b) == desc) { sh.list[i] = b; sh.list[j] = a; }
      }
      __syncthreads();
    }
  }
}

// With the list holding, sorted, every element of the kept set from the top
// down to at least the top-p cut: weights, their prefixes, and the top-p
// rule (an element stays while the mass strictly above its value is below
// X).  Returns (through sh) nkeep = the kept prefix length and the kept
// mass.  n = entries of the kept set held in the list; S_known = 0 means
// the list holds the whole kept set and its total is the kept mass.
__device__ int sv_list_top_p(SvShared& sh, int n, const SvWeight& W, bool top_p_on, float top_p,
                             uint64_t S_known, uint32_t& theta, uint64_t& S_final) {
  const int t = threadIdx.x;
  uint64_t w0 = 0, w1 = 0;
  if (2 * t < n) w0 = W(uint32_t(sh.list[2 * t] >> 32));
  if (2 * t + 1 < n) w1 = W(uint32_t(sh.list[2 * t + 1] >> 32));
  uint64_t ex = w0 + w1, dummy = 0, tot, tot2;
  sv_scan2(ex, dummy, tot, tot2, sh.scan);
  if (2 * t < n) sh.pre[2 * t] = ex;
  if (2 * t + 1 < n) sh.pre[2 * t + 1] = ex + w0;
  const uint64_t S = S_known ? S_known : tot;
  if (t == 0) sh.red[0] = uint32_t(n);
  __syncthreads();
  if (top_p_on) {
    const double X = double(top_p) * double(S);
    // keep flags are monotone along the list: the first dropped entry is
    // the kept length
    for (int j = t; j < n; j += SV_THREADS) {
      const uint32_t kj = uint32_t(sh.list[j] >> 32);
      int lo = 0, hi = j;  // first index whose key equals kj
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (uint32_t(sh.list[mid] >> 32) > kj) lo = mid + 1; else hi = mid;
      }
      if (!(double(sh.pre[lo]) < X)) atomicMin(&sh.red[0], uint32_t(j));
    }
    __syncthreads();
  }
  const int nkeep = int(sh.red[0]);
  theta = uint32_t(sh.list[nkeep - 1] >> 32);
  const uint64_t wl = W(theta);
  S_final = sh.pre[nkeep - 1] + wl;
  __syncthreads();
  return nkeep;
}

}  // namespace

// grid = B * bs rows, block = 1024.  Rows past a sequence's draft length
// plus one are skipped (never read).
__global__ __launch_bounds__(SV_THREADS) void sample_rows_kernel(SampleArgs p) {
  __shared__ SvShared sh;
  const int row = blockIdx.x;
  const int b = row / p.bs, i = row - b * p.bs;
  const int P = p.bs - 1;
  const int len = p.lens ? min(max(p.lens[b], 0), P) : P;
  if (i > len) return;
  const int V = p.V;
  const float* z = p.logits + int64_t(row) * V;
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0;
  const int t = threadIdx.x;

  const bool topk_on = p.top_k > 0;
  const bool top_p_on = p.top_p < 1.0f;
  bool in_list = false;      // the list holds the kept set from the top, sorted
  int nkept = V;             // size of the kept set (top-k)
  uint32_t tk = 0u;          // kept set = keys >= tk
  uint32_t mk = 0u;          // the row's largest key
  if (topk_on) {
    // ---- top-k in one pass over the row.  The first ns ids estimate where
    // the k largest end (the level-0 bin holding the sample's j-th largest,
    // j = k scaled to the sample plus a margin); the pass then takes the row
    // maximum and collects every element at or above that bin.  Exact
    // whenever at least k elements were collected (the k-th largest and all
    // its ties are then in the list) and they fit it; otherwise the exact
    // radix select below runs.
    const int ns = vec ? (min(V, max(4096, V / 16)) & ~3) : min(V, max(4096, V / 16));
    sv_clear(sh, false);
    sv_for_row(z, ns, vec, [&](int, float x) { atomicAdd(&sh.cnt[sv_key(sv_clean(x)) >> 21], 1u); });
    __syncthreads();
    const int target = min(ns, int((int64_t(p.top_k) * ns + V - 1) / V) + 8);
    sv_find(sh, SV_BINS, false, double(target), 0ull);
    const uint32_t lo = sh.fbin << 21;
    if (t == 0) sh.nlist = 0u;
    __syncthreads();
    sv_for_row(z, V, vec, [&](int id, float x) {
      const uint32_t k = sv_key(sv_clean(x));
      mk = k > mk ? k : mk;
      if (k >= lo) {
        const uint32_t slot = atomicAdd(&sh.nlist, 1u);
        if (slot < uint32_t(SV_CAP)) sh.list[slot] = (uint64_t(k) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(id));
      }
    });
  } else {
    // ---- row maximum
    sv_for_row(z, V, vec, [&](int, float x) {
      const uint32_t k = sv_key(sv_clean(x));
      mk = k > mk ? k : mk;
    });
  }
  {
    uint32_t v = mk;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t w = __shfl_xor(v, o, WAVE);
      v = w > v ? w : v;
    }
    if ((t & (WAVE - 1)) == 0) sh.red[t / WAVE] = v;
    __syncthreads();
    mk = 0u;
    for (int w = 0; w < SV_WAVES; ++w) mk = sh.red[w] > mk ? sh.red[w] : mk;
    __syncthreads();
  }
  SvWeight W;
  W.mkey = mk; W.m = sv_val(mk); W.temp = p.temp; W.qscale = p.qscale;
  if (topk_on) {
    const uint32_t n = sh.nlist;
    if (n >= uint32_t(p.top_k) && n <= uint32_t(SV_CAP)) {
      sv_sort(sh, int(n));
      tk = uint32_t(sh.list[p.top_k - 1] >> 32);
      if (t == 0) sh.red[0] = uint32_t(p.top_k);
      __syncthreads();
      for (int j = p.top_k + t; j < int(n); j += SV_THREADS)
        if (uint32_t(sh.list[j] >> 32) >= tk) atomicMax(&sh.red[0], uint32_t(j + 1));
      __syncthreads();
      nkept = int(sh.red[0]);
      __syncthreads();
      in_list = true;
    }
  }
  if (topk_on && !in_list) {
    uint32_t prefix = 0u;
    uint64_t base = 0ull;
    sv_hist(sh, z, V, vec, 0, 0u, 0u, nullptr);
    for (int level = 0; level < 3; ++level) {
      if (level > 0) sv_hist(sh, z, V, vec, level, prefix, 0u, nullptr);
      sv_find(sh, level == 2 ? 1024 : SV_BINS, false, double(p.top_k), base);
      const uint32_t bin = sh.fbin;
      const uint64_t above = sh.fabove_c, hbin = sh.fbin_c;
      __syncthreads();
      prefix = level == 0 ? bin : ((prefix << (level == 1 ? 11 : 10)) | bin);
      base += above;
      if (base + hbin <= uint64_t(SV_CAP)) {
        sv_collect(sh, z, V, vec, prefix << sv_shift(level));
        sv_sort(sh, int(base + hbin));
        tk = uint32_t(sh.list[min(p.top_k, int(base + hbin)) - 1] >> 32);
        // kept = list entries with key >= tk (the k-th and its ties)
        if (t == 0) sh.red[0] = uint32_t(p.top_k);
        __syncthreads();
        for (int j = p.top_k + t; j < int(base + hbin); j += SV_THREADS)
          if (uint32_t(sh.list[j] >> 32) >= tk) atomicMax(&sh.red[0], uint32_t(j + 1));
        __syncthreads();
        nkept = int(sh.red[0]);
        __syncthreads();
        in_list = true;
        break;
      }
      if (level == 2) {
        tk = prefix;
        nkept = int(base + hbin);
      }
    }
  } else if (!topk_on && V <= SV_CAP) {
    sv_collect(sh, z, V, vec, 0u);
    sv_sort(sh, V);
    in_list = true;
  }

  // ---- masses and top-p
  uint32_t theta;
  uint64_t S_final;
  int nlisted = 0;           // kept set held, sorted, in list[0, nlisted) (0: not held)
  if (in_list) {
    nlisted = sv_list_top_p(sh, nkept, W, top_p_on, p.top_p, 0ull, theta, S_final);
  } else {
    sv_hist(sh, z, V, vec, 0, 0u, tk, &W);
    if (!top_p_on) {
      // total kept mass: the scan inside sv_find sums every bin
      sv_find(sh, SV_BINS, true, 0.0, 0ull);
      theta = tk;
      S_final = sh.total_w;
      __syncthreads();
    } else {
      sv_find(sh, SV_BINS, true, 0.0, 0ull);
      const uint64_t S_K = sh.total_w;
      __syncthreads();
      const double X = double(p.top_p) * double(S_K);
      uint32_t prefix = 0u;
      uint64_t base_w = 0ull, base_c = 0ull;
      theta = tk;
      S_final = S_K;
      for (int level = 0; level < 3; ++level) {
        if (level > 0) sv_hist(sh, z, V, vec, level, prefix, tk, &W);
        sv_find(sh, level == 2 ? 1024 : SV_BINS, true, X, base_w);
        const uint32_t bin = sh.fbin;
        const uint64_t aw = sh.fabove_w, ac = sh.fabove_c, bw = sh.fbin_w, bc = sh.fbin_c;
        __syncthreads();
        prefix = level == 0 ? bin : ((prefix << (level == 1 ? 11 : 10)) | bin);
        base_w += aw;
        base_c += ac;
        if (base_c + bc <= uint64_t(SV_CAP)) {
          const uint32_t lo = prefix << sv_shift(level);
          sv_collect(sh, z, V, vec, lo > tk ? lo : tk);
          sv_sort(sh, int(base_c + bc));
          nlisted = sv_list_top_p(sh, int(base_c + bc), W, true, p.top_p, S_K, theta, S_final);
          break;
        }
        if (level == 2) {
          theta = prefix;
          S_final = base_w + bw;
        }
      }
    }
  }

  // hand a small kept set to the draw (ids and weights, value desc)
  const bool hand = nlisted > 0 && nlisted <= SV_OUT;
  if (hand) {
    for (int j = t; j < nlisted; j += SV_THREADS) {
      const uint64_t e = sh.list[j];
      p.kept_id[int64_t(row) * SV_OUT + j] = 0xFFFFFFFFu - uint32_t(e);
      p.kept_w[int64_t(row) * SV_OUT + j] = W(uint32_t(e >> 32));
    }
  }
  if (t == 0) {
    p.kept_n[row] = hand ? nlisted : 0;
    uint64_t Ed = 0ull;
    if (i < len) {
      const int d = p.drafts[int64_t(b) * P + i];
      if (d >= 0 && d < V) {
        const uint32_t kd = sv_key(sv_clean(z[d]));
        if (kd >= theta) Ed = W(kd);
      }
    }
    p.theta[row] = theta;
    p.mkey[row] = mk;
    p.S[row] = S_final;
    p.Ed[row] = Ed;
  }
}

// One block of 1024 per sequence: the accepted prefix, then the bonus draw.
// A kept set the row pass handed over (at most SV_OUT entries) is drawn from
// directly: entry j is the draw when the mass of the entries with ids <= its
// own first exceeds R.  Otherwise an exact fixed-point prefix scan walks the
// stop row in id order, 16 ids per thread per step.
__global__ __launch_bounds__(SV_THREADS) void sample_pick_kernel(SampleArgs p) {
  __shared__ uint64_t scan[2 * SV_WAVES];
  __shared__ uint32_t kid[SV_OUT];
  __shared__ uint64_t kw[SV_OUT];
  __shared__ int s_n, s_found;
  __shared__ uint64_t s_best;
  const int b = blockIdx.x, t = threadIdx.x;
  const int P = p.bs - 1;
  const int len = p.lens ? min(max(p.lens[b], 0), P) : P;
  const int64_t r0 = int64_t(b) * p.bs;
  if (t == 0) {
    int n = 0;
    while (n < len) {
      const double u = double(p.uni[r0 + n]);
      if (!(u * double(p.S[r0 + n]) < double(p.Ed[r0 + n]))) break;
      ++n;
    }
    s_n = n;
    s_found = -1;
    s_best = 0ull;
  }
  if (p.draft_prob) {
    for (int j = t; j < P; j += SV_THREADS)
      p.draft_prob[int64_t(b) * P + j] =
          j < len ? float(double(p.Ed[r0 + j]) / double(p.S[r0 + j])) : 0.0f;
  }
  __syncthreads();
  const int n = s_n;
  const int64_t row = r0 + n;
  const bool residual = n < len;
  const int d = residual ? p.drafts[int64_t(b) * P + n] : -1;
  const uint64_t S = p.S[row] - (residual ? p.Ed[row] : 0ull);
  double v = double(p.uni[r0 + P]);
  if (!(v >= 0.0)) v = 0.0;
  const double Rd = floor(v * double(S));
  const uint64_t R = Rd >= double(S) ? S : uint64_t(Rd);
  const int nk = p.kept_n[row];
  if (nk > 0) {
    if (t < nk) {
      const uint32_t id = p.kept_id[row * SV_OUT + t];
      kid[t] = id;
      kw[t] = id == uint32_t(d) ? 0ull : p.kept_w[row * SV_OUT + t];
    }
    __syncthreads();
    if (t < nk && kw[t] > 0ull) {
      const uint32_t me = kid[t];
      uint64_t cum = 0ull;
      for (int i = 0; i < nk; ++i) cum += kid[i] <= me ? kw[i] : 0ull;
      if (cum > R && cum - kw[t] <= R) s_found = int(me);
    }
    __syncthreads();
    if (t == 0 && s_found < 0) {
      // no draw (only for a uniform outside [0, 1)): the most likely
      // eligible id = the first in (value desc, id asc) order
      for (int i = 0; i < nk; ++i)
        if (kid[i] != uint32_t(d)) { s_best = (uint64_t(1) << 32) | uint64_t(0xFFFFFFFFu - kid[i]); break; }
    }
    __syncthreads();
  } else {
    const uint32_t theta = p.theta[row];
    SvWeight W;
    W.mkey = p.mkey[row]; W.m = sv_val(W.mkey); W.temp = p.temp; W.qscale = p.qscale;
    const int V = p.V;
    const float* z = p.logits + row * V;
    const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0;
    uint64_t running = 0ull, best = 0ull;
    for (int j0 = 0; j0 < V; j0 += 16 * SV_THREADS) {
      const int j = j0 + 16 * t;     // this thread's 16 consecutive ids
      float x[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int jj = j + 4 * u;
        if (vec && jj + 3 < V) {
          const f32x4 q = *reinterpret_cast<const f32x4*>(z + jj);
          x[4 * u] = q[0]; x[4 * u + 1] = q[1]; x[4 * u + 2] = q[2]; x[4 * u + 3] = q[3];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * u + e] = jj + e < V ? z[jj + e] : -INFINITY;
        }
      }
      uint64_t s = 0ull;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t k = sv_key(sv_clean(x[e]));
        const bool elig = j + e < V && j + e != d && k >= theta;
        s += elig ? W(k) : 0ull;
        if (elig) {
          const uint64_t rk = (uint64_t(k) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(j + e));
          best = rk > best ? rk : best;
        }
      }
      uint64_t ex = s, dummy = 0ull, tot, tot2;
      sv_scan2(ex, dummy, tot, tot2, scan);
      const uint64_t c0 = running + ex;
      if (c0 <= R && R < c0 + s) {
        uint64_t c = c0;
        for (int e = 0; e < 16; ++e) {
          const uint32_t k = sv_key(sv_clean(x[e]));
          const bool elig = j + e < V && j + e != d && k >= theta;
          c += elig ? W(k) : 0ull;
          if (c > R) { s_found = j + e; break; }
        }
      }
      running += tot;
      __syncthreads();
      if (s_found >= 0) break;
    }
    if (s_found < 0) {
      // no draw (only for a uniform outside [0, 1)): the most likely eligible id
      atomicMax(reinterpret_cast<unsigned long long*>(&s_best), (unsigned long long)best);
      __syncthreads();
    }
  }
  if (t == 0) {
    int g = s_found;
    if (g < 0) g = s_best ? int(0xFFFFFFFFu - uint32_t(s_best)) : (d >= 0 ? d : 0);
    p.accepted[b] = n;
    p.bonus[b] = g;
  }
}

void launch_sample_rows(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sample_rows_kernel, dim3(a.B * a.bs), dim3(SV_THREADS), 0, s, a);
}

void launch_sample_pick(const SampleArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(sample_pick_kernel, dim3(a.B), dim3(SV_THREADS), 0, s, a);
}

}  // namespace dfl

// Row-wise kernels of the draft step: residual update + in-block
// convolution + RMSNorm, the QKV epilogue (split-K reduction, RoPE, cache
// writes), the context-append epilogue and SwiGLU.  All are small and bound
// by launch latency or by one pass over their rows; each fuses the
// reduction of the preceding GEMM's split-K partial sums (fixed order, so
// results are deterministic).
#include "common.h"
#include "kernels.h"

namespace dfl {

// Sum of the split-K partial sums of one element, s = 0, 1, ... in order.
// Loads are issued eight at a time so their latencies overlap.
__device__ __forceinline__ float sum_parts(const float* __restrict__ parts, int splits, int64_t ss,
                                           int64_t idx) {
  float v = 0.f;
  int s = 0;
  for (; s + 8 <= splits; s += 8) {
    float t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = parts[(s + u) * ss + idx];
#pragma unroll
    for (int u = 0; u < 8; ++u) v += t[u];
  }
  if (s + 4 <= splits) {
    float t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = parts[(s + u) * ss + idx];
#pragma unroll
    for (int u = 0; u < 4; ++u) v += t[u];
    s += 4;
  }
  for (; s < splits; ++s) v += parts[s * ss + idx];
  return v;
}

// Four consecutive elements of an activation row (16 or 8 bytes, aligned:
// every row length here is a multiple of 32).
template <typename T> struct Act4;
template <> struct Act4<float> {
  __device__ static f32x4 load(const float* p, int64_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
  __device__ static void store(float* p, int64_t i, f32x4 v) { *reinterpret_cast<f32x4*>(p + i) = v; }
};
template <> struct Act4<bf16_t> {
  __device__ static f32x4 load(const bf16_t* p, int64_t i) {
    const uint2 u = *reinterpret_cast<const uint2*>(p + i);
    return f32x4{bf16_to_f32(bf16_t(u.x & 0xFFFFu)), bf16_to_f32(bf16_t(u.x >> 16)),
                 bf16_to_f32(bf16_t(u.y & 0xFFFFu)), bf16_to_f32(bf16_t(u.y >> 16))};
  }
  __device__ static void store(bf16_t* p, int64_t i, f32x4 v) {
    uint2 u;
    u.x = f32x2_to_bf16x2(v[0], v[1]);
    u.y = f32x2_to_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p + i) = u;
  }
};

// sum_parts for four consecutive elements (16-byte loads, four splits in
// flight, splits added in order).
__device__ __forceinline__ f32x4 sum_parts4(const float* __restrict__ parts, int splits, int64_t ss,
                                            int64_t idx) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= splits; s += 4) {
    f32x4 t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = *reinterpret_cast<const f32x4*>(parts + (s + u) * ss + idx);
#pragma unroll
    for (int u = 0; u < 4; ++u) v += t[u];
  }
  for (; s < splits; ++s) v += *reinterpret_cast<const f32x4*>(parts + s * ss + idx);
  return v;
}

// VEC consecutive elements (VEC = 1 or 4) of an activation / float row.
__host__ __device__ inline int norm_col_blocks_dev(int H) { return (H + 255) / 256; }

template <typename T, int VEC> struct Vec;
template <typename T> struct Vec<T, 4> {
  typedef f32x4 V;
  __device__ static V act(const T* p, int64_t i) { return Act4<T>::load(p, i); }
  __device__ static void put(T* p, int64_t i, V v) { Act4<T>::store(p, i, v); }
  __device__ static V f32(const float* p, int64_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
  __device__ static void putf(float* p, int64_t i, V v) { *reinterpret_cast<f32x4*>(p + i) = v; }
  __device__ static V parts(const float* p, int s, int64_t ss, int64_t i) { return sum_parts4(p, s, ss, i); }
  __device__ static V splat(float x) { return f32x4{x, x, x, x}; }
  __device__ static float sq(V y) { return ((y[0] * y[0] + y[1] * y[1]) + y[2] * y[2]) + y[3] * y[3]; }
};
template <typename T> struct Vec<T, 1> {
  typedef f32x1 V;
  __device__ static V act(const T* p, int64_t i) { return V{Act<T>::load(p, i)}; }
  __device__ static void put(T* p, int64_t i, V v) { Act<T>::store(p, i, v[0]); }
  __device__ static V f32(const float* p, int64_t i) { return V{p[i]}; }
  __device__ static void putf(float* p, int64_t i, V v) { p[i] = v[0]; }
  __device__ static V parts(const float* p, int s, int64_t ss, int64_t i) { return V{sum_parts(p, s, ss, i)}; }
  __device__ static V splat(float x) { return V{x}; }
  __device__ static float sq(V y) { return y[0] * y[0]; }
};

// block = 256 threads, VEC consecutive columns per thread: grid = (rows,
// ceil(H / (256 VEC))).  One element per thread for few rows, where latency
// rules; four for many rows, where bandwidth does (a wave then covers one
// 256-column block of the sums of squares).  Row r is slot t = r % bs of
// block b = r / bs.
//   input  h_in[r] = emb_scale * E[token]           (embedding mode)
//                  = base[r] + sum_s parts[s][r]      (residual mode)
//   conv   y[r]    = h_in[r] + sum_{j < conv_k, t - j >= 0} conv[j] * h_in[r - j]
//          (dynamic: conv[j] -> the slot's own tap j of the channel's group,
//          summed from the tap GEMM's split-K partials)
//   outputs h_out[r] = y[r];  n_out[o] = gain * y[r];  sumsq[o][col block] = sum y^2
// for output row o = b * (bs - t_first) + t - t_first when t >= t_first, one
// sum of squares per 256 columns.
// The RMSNorm factor 1/rms(y) is one scalar per row, so the consuming GEMM
// applies it to its result (GemmArgs.rs); n_out * W^T * (1/rms) equals
// RMSNorm(y) * W^T.  The in-block convolution is the DFlash 2 addition of the
// NeMo AutoModel page ("Variants" table); RMSNorm is the draft's norm.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void resconv_kernel(NormArgs p) {
  typedef Vec<T, VEC> X;
  typedef typename X::V V;
  __shared__ float red[16];
  const int rows = p.rows_dev ? min(*p.rows_dev, p.rows) : p.rows;
  int r = blockIdx.x, cb = blockIdx.y;
  if (p.remap_cb > 0) {
    // blocks go to the 8 XCDs round-robin; XCD x runs tiles [x per, (x + 1) per)
    // with the column block fastest, so the neighbour rows the convolution
    // reads were just loaded into the same L2
    const int per = int(gridDim.x >> 3);
    const int g = int(blockIdx.x & 7) * per + int(blockIdx.x >> 3);
    r = g / p.remap_cb;
    cb = g - r * p.remap_cb;
    if (r >= p.rows) return;
  }
  if (r >= rows) return;
  const int t = r % p.bs, b = r / p.bs;
  const int H = p.H;
  const int c = (cb * blockDim.x + threadIdx.x) * VEC;
  const T* E = static_cast<const T*>(p.embed);
  const T* C = static_cast<const T*>(p.conv);

  auto hin = [&](int rr) -> V {
    if (E) {
      const int tt = rr % p.bs;
      const int tok = tt == 0 ? p.anchors[rr / p.bs] : p.mask_id;
      if (tok < 0 || tok >= p.vocab) return X::splat(0.f);
      return p.emb_scale * X::act(E, int64_t(tok) * H + c);
    }
    V v = p.base ? X::f32(p.base, int64_t(rr) * H + c) : X::splat(0.f);
    if (p.parts) v += X::parts(p.parts, p.splits, p.split_stride, int64_t(rr) * p.ldp + c);
    return v;
  };

  V y = X::splat(0.f);
  if (c < H) {
    y = hin(r);
    if (C) {
      const V x0 = y;
      y = x0 + X::act(C, c) * x0;
      for (int j = 1; j < p.conv_k && t - j >= 0; ++j) y += X::act(C, int64_t(j) * H + c) * hin(r - j);
    } else if (p.dtaps) {
      // dynamic taps of this slot, shared by each channel's group
      int64_t trow[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) trow[e] = int64_t(r) * p.dgk + int64_t((c + e) / p.dgroup) * p.conv_k;
      const V x0 = y;
#pragma unroll
      for (int e = 0; e < VEC; ++e) y[e] = x0[e] + sum_parts(p.dtaps, p.dsplits, p.dstride, trow[e]) * x0[e];
      for (int j = 1; j < p.conv_k && t - j >= 0; ++j) {
        const V xj = hin(r - j);
#pragma unroll
        for (int e = 0; e < VEC; ++e) y[e] += sum_parts(p.dtaps, p.dsplits, p.dstride, trow[e] + j) * xj[e];
      }
    }
    if (p.h_out) X::putf(p.h_out, int64_t(r) * H + c, y);
  }
  if (t < p.t_first) return;  // uniform per block
  const int orow = b * (p.bs - p.t_first) + (t - p.t_first);
  if (c < H) {
    const V g = p.gain ? X::act(static_cast<const T*>(p.gain), c) : X::splat(1.f);
    X::put(static_cast<T*>(p.n_out), int64_t(orow) * H + c, y * g);
  }
  const int nslots = norm_col_blocks_dev(H);
  if (VEC == 1) {
    const float ss = block_sum(X::sq(y), red);
    if (threadIdx.x == 0) p.sumsq[int64_t(orow) * nslots + cb] = ss;
  } else {
    const float ss = wave_sum(X::sq(y));
    const int slot = cb * (256 * VEC / 256) + int(threadIdx.x) / WAVE;
    if ((threadIdx.x & (WAVE - 1)) == 0 && slot < nslots) p.sumsq[int64_t(orow) * nslots + slot] = ss;
  }
}

// Rotate-half RoPE: pair i of a head of width d at position pos turns by the
// angle pos * theta^(-2 i / d).  The frequencies, i < d / 2, in double, one
// table per block (d <= 256).
__device__ __forceinline__ void rope_table(double* inv_freq, int d, float theta) {
  for (int i = threadIdx.x; i < d / 2; i += blockDim.x)
    inv_freq[i] = pow(double(theta), -2.0 * double(i) / double(d));
  __syncthreads();
}

// cos and sin of pos * inv: float32 activations take the double sine and
// cosine; bf16 ones the angle reduced to [-pi, pi] in double, then the
// hardware sine and cosine (~1e-6 absolute error, far below bf16 rounding).
// With the per-block frequency table this took the batched workload's QKV
// epilogue from 21.6 to 15.6 us (a double pow and sine/cosine per pair before).
template <typename T>
__device__ __forceinline__ void rope_cs_t(int pos, double inv, float& c, float& s) {
  if constexpr (sizeof(T) == 4) {
    double sn, cs;
    sincos(double(pos) * inv, &sn, &cs);
    c = float(cs);
    s = float(sn);
  } else {
    const double ang = double(pos) * inv;
    const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    __sincosf(float(red), &s, &c);
  }
}

// grid = (M rows, nq + 2 nkv heads), block = 64.  Slot t of block b sits at
// position ctx_lens[b] + t.  q heads -> q_out; k heads (after RoPE) and v
// heads -> the cache rows [L_b, L_b + bs) of this layer (V transposed).
template <typename T>
__global__ __launch_bounds__(64) void qkv_epilogue_kernel(QkvEpiArgs p) {
  __shared__ double inv_freq[128];
  rope_table(inv_freq, p.d, p.theta);
  const int m = blockIdx.x, h = blockIdx.y;
  const int b = m / p.bs, t = m % p.bs;
  const int pos = p.ctx_lens[b] + t;
  const int d = p.d, half = d / 2;
  const int64_t row = int64_t(m) * p.ldp + int64_t(h) * d;
  T* q = static_cast<T*>(p.q_out);
  T* kc = static_cast<T*>(p.k_layer);
  T* vc = static_cast<T*>(p.v_layer);
  const bool in_cache = pos >= 0 && pos < p.Lmax;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float x0 = sum_parts(p.parts, p.splits, p.split_stride, row + i);
    float x1 = sum_parts(p.parts, p.splits, p.split_stride, row + i + half);
    if (h < p.nq + p.nkv) {
      float c, s;
      rope_cs_t<T>(pos, inv_freq[i], c, s);
      const float y0 = x0 * c - x1 * s;
      const float y1 = x1 * c + x0 * s;
      x0 = y0;
      x1 = y1;
    }
    if (h < p.nq) {
      const int64_t o = (int64_t(m) * p.nq + h) * d;
      Act<T>::store(q, o + i, x0);
      Act<T>::store(q, o + i + half, x1);
    } else if (in_cache) {
      if (h < p.nq + p.nkv) {
        const int g = h - p.nq;
        const int64_t o = ((int64_t(b) * p.nkv + g) * p.Lmax + pos) * d;
        Act<T>::store(kc, o + i, x0);
        Act<T>::store(kc, o + i + half, x1);
      } else {
        const int g = h - p.nq - p.nkv;
        const int64_t o = (int64_t(b) * p.nkv + g) * d * p.Lmax + pos;
        Act<T>::store(vc, o + int64_t(i) * p.Lmax, x0);
        Act<T>::store(vc, o + int64_t(i + half) * p.Lmax, x1);
      }
    }
  }
}

// Wide variant of qkv_epilogue_kernel: four consecutive pairs per thread
// (16-byte partial loads), half / 4 threads per head, 64 / (half / 4) heads
// per block of 64; grid = (M rows, ceil(heads / heads per block)).
template <typename T>
__global__ __launch_bounds__(64) void qkv_epilogue4_kernel(QkvEpiArgs p) {
  __shared__ double inv_freq[128];
  rope_table(inv_freq, p.d, p.theta);   // before any thread leaves
  const int d = p.d, half = d / 2, tph = half / 4, hpb = 64 / tph;
  const int m = blockIdx.x;
  const int h = blockIdx.y * hpb + int(threadIdx.x) / tph;
  const int i = (int(threadIdx.x) % tph) * 4;
  if (h >= p.nq + 2 * p.nkv) return;
  const int b = m / p.bs, t = m % p.bs;
  const int pos = p.ctx_lens[b] + t;
  const int64_t row = int64_t(m) * p.ldp + int64_t(h) * d;
  T* q = static_cast<T*>(p.q_out);
  T* kc = static_cast<T*>(p.k_layer);
  T* vc = static_cast<T*>(p.v_layer);
  f32x4 x0 = sum_parts4(p.parts, p.splits, p.split_stride, row + i);
  f32x4 x1 = sum_parts4(p.parts, p.splits, p.split_stride, row + i + half);
  if (h < p.nq + p.nkv) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float c, sn;
      rope_cs_t<T>(pos, inv_freq[i + e], c, sn);
      const float y0 = x0[e] * c - x1[e] * sn;
      const float y1 = x1[e] * c + x0[e] * sn;
      x0[e] = y0;
      x1[e] = y1;
    }
  }
  if (h < p.nq) {
    const int64_t o = (int64_t(m) * p.nq + h) * d;
    Act4<T>::store(q, o + i, x0);
    Act4<T>::store(q, o + i + half, x1);
  } else if (pos >= 0 && pos < p.Lmax) {
    if (h < p.nq + p.nkv) {
      const int g = h - p.nq;
      const int64_t o = ((int64_t(b) * p.nkv + g) * p.Lmax + pos) * d;
      Act4<T>::store(kc, o + i, x0);
      Act4<T>::store(kc, o + i + half, x1);
    } else {
      const int g = h - p.nq - p.nkv;
      const int64_t o = (int64_t(b) * p.nkv + g) * d * p.Lmax + pos;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Act<T>::store(vc, o + int64_t(i + e) * p.Lmax, x0[e]);
        Act<T>::store(vc, o + int64_t(i + e + half) * p.Lmax, x1[e]);
      }
    }
  }
}

// grid = (Mn rows, nL * 2 nkv), block = 64.  New context row r belongs to the
// sequence b with offsets[b] <= r < offsets[b + 1] and sits at position
// ctx_lens[b] - n_b + (r - offsets[b]).
template <typename T>
__global__ __launch_bounds__(64) void kv_append_kernel(KvAppendArgs p) {
  const int Mact = min(p.offsets[p.B], p.Mn);
  const int r = blockIdx.x;
  if (r >= Mact) return;
  int lo = 0, hi = p.B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.offsets[mid] <= r) lo = mid; else hi = mid;
  }
  const int b = lo;
  const int nb = p.offsets[b + 1] - p.offsets[b];
  const int pos = p.ctx_lens[b] - nb + (r - p.offsets[b]);
  if (pos < 0 || pos >= p.Lmax) return;
  const int l = blockIdx.y / (2 * p.nkv), hh = blockIdx.y % (2 * p.nkv);
  const int d = p.d, half = d / 2;
  __shared__ double inv_freq[128];
  rope_table(inv_freq, d, p.theta);   // (the returns above are block-uniform)
  const float* parts = p.parts + int64_t(l) * p.layer_stride;
  const int64_t row = int64_t(r) * p.ldp + int64_t(hh) * d;
  T* kc = static_cast<T*>(p.k_cache) + int64_t(l) * p.cache_layer_stride;
  T* vc = static_cast<T*>(p.v_cache) + int64_t(l) * p.cache_layer_stride;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float x0 = sum_parts(parts, p.splits, p.split_stride, row + i);
    float x1 = sum_parts(parts, p.splits, p.split_stride, row + i + half);
    if (hh < p.nkv) {
      float c, s;
      rope_cs_t<T>(pos, inv_freq[i], c, s);
      const int64_t o = ((int64_t(b) * p.nkv + hh) * p.Lmax + pos) * d;
      Act<T>::store(kc, o + i, x0 * c - x1 * s);
      Act<T>::store(kc, o + i + half, x1 * c + x0 * s);
    } else {
      const int g = hh - p.nkv;
      const int64_t o = (int64_t(b) * p.nkv + g) * d * p.Lmax + pos;
      Act<T>::store(vc, o + int64_t(i) * p.Lmax, x0);
      Act<T>::store(vc, o + int64_t(i + half) * p.Lmax, x1);
    }
  }
}

// act[m][f] = SiLU(gate) * up, gate = row m col f, up = col F + f; VEC
// consecutive f per thread (F is a multiple of 32).
template <typename T, int VEC>
__global__ __launch_bounds__(256) void swiglu_kernel(SwigluArgs p) {
  typedef Vec<T, VEC> X;
  const int64_t idx = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * VEC;
  if (idx >= int64_t(p.M) * p.F) return;
  const int m = int(idx / p.F), f = int(idx % p.F);
  const int64_t base = int64_t(m) * p.ldp;
  const typename X::V gt = X::parts(p.parts, p.splits, p.split_stride, base + f);
  const typename X::V up = X::parts(p.parts, p.splits, p.split_stride, base + p.F + f);
  typename X::V y;
#pragma unroll
  for (int e = 0; e < VEC; ++e) y[e] = gt[e] / (1.0f + expf(-gt[e])) * up[e];
  X::put(static_cast<T*>(p.out), idx, y);
}

int norm_col_blocks(int H) { return norm_col_blocks_dev(H); }

void launch_norm(bool f32, const NormArgs& a0, hipStream_t s) {
  // few rows: one element per thread (more blocks, shorter chains); many
  // rows: four per thread (16-byte accesses), tiles dealt to the XCDs in
  // contiguous runs
  NormArgs a = a0;
  const bool wide = a.rows > 64;
  const int cbs = wide ? (a.H + 1023) / 1024 : norm_col_blocks(a.H);
  const int64_t tiles = int64_t(a.rows) * cbs;
  a.remap_cb = (wide && tiles < (int64_t(1) << 30)) ? cbs : 0;
  const dim3 grid = a.remap_cb ? dim3(unsigned((tiles + 7) / 8 * 8)) : dim3(a.rows, cbs);
  if (f32) {
    if (wide) hipLaunchKernelGGL((resconv_kernel<float, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((resconv_kernel<float, 1>), grid, dim3(256), 0, s, a);
  } else {
    if (wide) hipLaunchKernelGGL((resconv_kernel<bf16_t, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((resconv_kernel<bf16_t, 1>), grid, dim3(256), 0, s, a);
  }
}

void launch_qkv_epilogue(bool f32, const QkvEpiArgs& a, hipStream_t s) {
  if (a.M > 64) {
    // many rows: four pairs per thread, 16-byte partial loads
    const int hpb = 64 / (a.d / 8);
    const dim3 grid(a.M, (a.nq + 2 * a.nkv + hpb - 1) / hpb);
    if (f32) hipLaunchKernelGGL(qkv_epilogue4_kernel<float>, grid, dim3(64), 0, s, a);
    else hipLaunchKernelGGL(qkv_epilogue4_kernel<bf16_t>, grid, dim3(64), 0, s, a);
    return;
  }
  dim3 grid(a.M, a.nq + 2 * a.nkv);
  if (f32) hipLaunchKernelGGL(qkv_epilogue_kernel<float>, grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL(qkv_epilogue_kernel<bf16_t>, grid, dim3(64), 0, s, a);
}

void launch_kv_append(bool f32, const KvAppendArgs& a, hipStream_t s) {
  dim3 grid(a.Mn, a.nL * 2 * a.nkv);
  if (f32) hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(64), 0, s, a);
  else hipLaunchKernelGGL(kv_append_kernel<bf16_t>, grid, dim3(64), 0, s, a);
}

void launch_swiglu(bool f32, const SwigluArgs& a, hipStream_t s) {
  const int64_t n = int64_t(a.M) * a.F;
  const bool wide = a.M > 64;
  const dim3 grid(unsigned(wide ? (n / 4 + 255) / 256 : (n + 255) / 256));
  if (f32) {
    if (wide) hipLaunchKernelGGL((swiglu_kernel<float, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((swiglu_kernel<float, 1>), grid, dim3(256), 0, s, a);
  } else {
    if (wide) hipLaunchKernelGGL((swiglu_kernel<bf16_t, 4>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((swiglu_kernel<bf16_t, 1>), grid, dim3(256), 0, s, a);
  }
}

}  // namespace dfl

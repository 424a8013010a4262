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

// grid = (rows, ceil(H / 256)), one thread per (row, column).  Row r is slot
// t = r % bs of block b = r / bs.
//   input  h_in[r] = emb_scale * E[token]           (embedding mode)
//                  = base[r] + sum_s parts[s][r]      (residual mode)
//   conv   y[r]    = h_in[r] + sum_{j < conv_k, t - j >= 0} conv[j] * h_in[r - j]
//          (dynamic: conv[j] -> the slot's own tap j of the channel's group,
//          summed from the tap GEMM's split-K partials)
//   outputs h_out[r] = y[r];  n_out[o] = gain * y[r];  sumsq[o][col block] = sum y^2
// for output row o = b * (bs - t_first) + t - t_first when t >= t_first.
// The RMSNorm factor 1/rms(y) is one scalar per row, so the consuming GEMM
// applies it to its result (GemmArgs.rs); n_out * W^T * (1/rms) equals
// RMSNorm(y) * W^T.  The in-block convolution is the DFlash 2 addition of the
// NeMo AutoModel page ("Variants" table); RMSNorm is the draft's norm.
template <typename T>
__global__ __launch_bounds__(256) void resconv_kernel(NormArgs p) {
  __shared__ float red[16];
  const int rows = p.rows_dev ? min(*p.rows_dev, p.rows) : p.rows;
  const int r = blockIdx.x;
  if (r >= rows) return;
  const int t = r % p.bs, b = r / p.bs;
  const int H = p.H;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  const T* E = static_cast<const T*>(p.embed);
  const T* C = static_cast<const T*>(p.conv);

  auto hin = [&](int rr) -> float {
    if (E) {
      const int tt = rr % p.bs;
      const int tok = tt == 0 ? p.anchors[rr / p.bs] : p.mask_id;
      if (tok < 0 || tok >= p.vocab) return 0.f;
      return p.emb_scale * Act<T>::load(E, int64_t(tok) * H + c);
    }
    float v = p.base ? p.base[int64_t(rr) * H + c] : 0.f;
    if (p.parts) v += sum_parts(p.parts, p.splits, p.split_stride, int64_t(rr) * p.ldp + c);
    return v;
  };

  float y = 0.f;
  if (c < H) {
    y = hin(r);
    if (C) {
      const float x0 = y;
      y = x0 + Act<T>::load(C, c) * x0;
      for (int j = 1; j < p.conv_k && t - j >= 0; ++j) y += Act<T>::load(C, int64_t(j) * H + c) * hin(r - j);
    } else if (p.dtaps) {
      // dynamic taps of this slot, shared by the channel group of c
      const int64_t trow = int64_t(r) * p.dgk + int64_t(c / p.dgroup) * p.conv_k;
      const float x0 = y;
      y = x0 + sum_parts(p.dtaps, p.dsplits, p.dstride, trow) * x0;
      for (int j = 1; j < p.conv_k && t - j >= 0; ++j)
        y += sum_parts(p.dtaps, p.dsplits, p.dstride, trow + j) * hin(r - j);
    }
    if (p.h_out) p.h_out[int64_t(r) * H + c] = y;
  }
  if (t < p.t_first) return;  // uniform per block
  const int orow = b * (p.bs - p.t_first) + (t - p.t_first);
  if (c < H) {
    const float g = p.gain ? Act<T>::load(static_cast<const T*>(p.gain), c) : 1.0f;
    Act<T>::store(static_cast<T*>(p.n_out), int64_t(orow) * H + c, y * g);
  }
  const float ss = block_sum(y * y, red);
  if (threadIdx.x == 0) p.sumsq[int64_t(orow) * gridDim.y + blockIdx.y] = ss;
}

// Rotate-half RoPE angle for pair i of a head of width d at position pos,
// evaluated in double precision.
__device__ __forceinline__ void rope_cs(int pos, int i, int d, float theta, float& c, float& s) {
  const double inv = pow(double(theta), -2.0 * double(i) / double(d));
  double sn, cs;
  sincos(double(pos) * inv, &sn, &cs);
  c = float(cs);
  s = float(sn);
}

// grid = (M rows, nq + 2 nkv heads), block = 64.  Slot t of block b sits at
// position ctx_lens[b] + t.  q heads -> q_out; k heads (after RoPE) and v
// heads -> the cache rows [L_b, L_b + bs) of this layer (V transposed).
template <typename T>
__global__ __launch_bounds__(64) void qkv_epilogue_kernel(QkvEpiArgs p) {
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
      rope_cs(pos, i, d, p.theta, c, s);
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
  const float* parts = p.parts + int64_t(l) * p.layer_stride;
  const int64_t row = int64_t(r) * p.ldp + int64_t(hh) * d;
  T* kc = static_cast<T*>(p.k_cache) + int64_t(l) * p.cache_layer_stride;
  T* vc = static_cast<T*>(p.v_cache) + int64_t(l) * p.cache_layer_stride;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float x0 = sum_parts(parts, p.splits, p.split_stride, row + i);
    float x1 = sum_parts(parts, p.splits, p.split_stride, row + i + half);
    if (hh < p.nkv) {
      float c, s;
      rope_cs(pos, i, d, p.theta, c, s);
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

// act[m][f] = SiLU(gate) * up, gate = row m col f, up = col F + f.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_kernel(SwigluArgs p) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(p.M) * p.F) return;
  const int m = int(idx / p.F), f = int(idx % p.F);
  const int64_t base = int64_t(m) * p.ldp;
  const float gt = sum_parts(p.parts, p.splits, p.split_stride, base + f);
  const float up = sum_parts(p.parts, p.splits, p.split_stride, base + p.F + f);
  Act<T>::store(static_cast<T*>(p.out), idx, gt / (1.0f + expf(-gt)) * up);
}

int norm_col_blocks(int H) { return (H + 255) / 256; }

void launch_norm(bool f32, const NormArgs& a, hipStream_t s) {
  dim3 grid(a.rows, norm_col_blocks(a.H));
  if (f32) hipLaunchKernelGGL(resconv_kernel<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(resconv_kernel<bf16_t>, grid, dim3(256), 0, s, a);
}

void launch_qkv_epilogue(bool f32, const QkvEpiArgs& a, hipStream_t s) {
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
  dim3 grid(unsigned((n + 255) / 256));
  if (f32) hipLaunchKernelGGL(swiglu_kernel<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(swiglu_kernel<bf16_t>, grid, dim3(256), 0, s, a);
}

}  // namespace dfl

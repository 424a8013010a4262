// Path selector and greedy verification.
//
// Selector (NeMo AutoModel page, "Variants": a pairwise path selector walks
// one coherent path through each position's top-k candidates; "Objective":
// candidates are scored against the predecessor): one wavefront per
// sequence.  Per transition the factor-table rows of the previous and the
// current candidates are staged in LDS, all k*k pair scores are computed in
// float32 with separate multiply and add (m ascending), and a max-sum
// (Viterbi) step keeps the smallest predecessor on ties; the path is then
// traced back.  Only the listed order of float32 operations is used, so the
// result is bit-identical to any other evaluation in that order.
//
// Verification (NeMo SpeechLM page, "Validation"; llama-cpp-python wiki,
// "Prerequisites"): a row-wise argmax over the target logits, split into
// chunks so the whole logit tensor streams through HBM once, then a tiny
// kernel merges the chunks and finds the longest accepted prefix.
#include "common.h"
#include "kernels.h"

namespace dfl {

// This file is compiled with -ffp-contract=off: every product below is
// rounded before it is added, and each pair's sum runs over m in order.
// Rows are padded to RS = r rounded up to 4 floats (+4) so they can be read
// 16 bytes at a time from LDS; four pairs are accumulated side by side.
__device__ __forceinline__ void pair_dot4(const float* __restrict__ a0, const float* __restrict__ a1,
                                          const float* __restrict__ a2, const float* __restrict__ a3,
                                          const float* __restrict__ b0, const float* __restrict__ b1,
                                          const float* __restrict__ b2, const float* __restrict__ b3,
                                          int r, float (&out)[4]) {
  float c0 = 0.0f, c1 = 0.0f, c2 = 0.0f, c3 = 0.0f;
  int m = 0;
  for (; m + 4 <= r; m += 4) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(a0 + m), y0 = *reinterpret_cast<const f32x4*>(b0 + m);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(a1 + m), y1 = *reinterpret_cast<const f32x4*>(b1 + m);
    const f32x4 x2 = *reinterpret_cast<const f32x4*>(a2 + m), y2 = *reinterpret_cast<const f32x4*>(b2 + m);
    const f32x4 x3 = *reinterpret_cast<const f32x4*>(a3 + m), y3 = *reinterpret_cast<const f32x4*>(b3 + m);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = x0[e] * y0[e], p1 = x1[e] * y1[e], p2 = x2[e] * y2[e], p3 = x3[e] * y3[e];
      c0 = c0 + p0;
      c1 = c1 + p1;
      c2 = c2 + p2;
      c3 = c3 + p3;
    }
  }
  for (; m < r; ++m) {
    const float p0 = a0[m] * b0[m], p1 = a1[m] * b1[m], p2 = a2[m] * b2[m], p3 = a3[m] * b3[m];
    c0 = c0 + p0;
    c1 = c1 + p1;
    c2 = c2 + p2;
    c3 = c3 + p3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

__host__ __device__ int select_row_stride(int r) { return (r + 3) / 4 * 4 + 4; }

// LDS layout: tl_rows [k][RS], tr_rows [k][RS], pair [k][k], S [k],
// back [P][k] (int32).
__global__ __launch_bounds__(64) void select_kernel(SelectArgs p) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int k = p.k, r = p.r, P = p.P, rs = select_row_stride(r);
  float* TL = lds;
  float* TR = TL + k * rs;
  float* PAIR = TR + k * rs;
  float* S = PAIR + k * k;
  int32_t* BACK = reinterpret_cast<int32_t*>(S + k);
  const int32_t* ids = p.ids + int64_t(b) * P * k;
  const float* vals = p.vals + int64_t(b) * P * k;
  const int V = p.V;

  // Rows of `table` for the n candidate ids (n <= 64): the ids are read once
  // (one per lane) and shared through a shuffle; table loads go out eight at a time.
  auto stage = [&](float* dst, const float* table, const int32_t* src_ids, int n) {
    const int my_tok = lane < n ? src_ids[lane] : -1;
    for (int idx0 = 0; idx0 < n * r; idx0 += 8 * WAVE) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = idx0 + u * WAVE + lane;
        const int i = idx / r, m = idx - i * r;
        const int tok = __shfl(my_tok, i < n ? i : 0, WAVE);
        v[u] = (idx < n * r && tok >= 0 && tok < V) ? table[int64_t(tok) * r + m] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int idx = idx0 + u * WAVE + lane;
        const int i = idx / r, m = idx - i * r;
        if (idx < n * r) dst[i * rs + m] = v[u];
      }
    }
  };

  for (int t = 0; t < P; ++t) {
    // previous candidates: the anchor for t = 0
    if (t == 0) stage(TL, p.tl, p.anchors + b, 1);
    else stage(TL, p.tl, ids + (t - 1) * k, k);
    stage(TR, p.tr, ids + t * k, k);
    __syncthreads();
    const int nprev = t == 0 ? 1 : k;
    const int npairs = nprev * k;
    for (int q0 = lane; q0 < npairs; q0 += 4 * WAVE) {
      int qi[4];
      const float* ap[4];
      const float* bp[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        qi[u] = q0 + u * WAVE;
        const int qq = qi[u] < npairs ? qi[u] : q0;
        ap[u] = TL + (qq / k) * rs;
        bp[u] = TR + (qq % k) * rs;
      }
      float out[4];
      pair_dot4(ap[0], ap[1], ap[2], ap[3], bp[0], bp[1], bp[2], bp[3], r, out);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (qi[u] < npairs) PAIR[qi[u]] = out[u];
    }
    __syncthreads();
    if (p.debug_pair) {
      float* dp = p.debug_pair + (int64_t(b) * P + t) * k * k;
      for (int idx = lane; idx < k * k; idx += WAVE) {
        const int i = idx / k, j = idx % k;
        dp[idx] = PAIR[(t == 0 ? 0 : i) * k + j];
      }
    }
    float snew = 0.f;
    int bi = 0;
    if (lane < k) {
      const int j = lane;
      if (t == 0) {
        snew = PAIR[j] + vals[j];
      } else {
        float bv = S[0] + PAIR[j];
        for (int i = 1; i < k; ++i) {
          const float v = S[i] + PAIR[i * k + j];
          if (v > bv) { bv = v; bi = i; }
        }
        snew = bv + vals[t * k + j];
      }
    }
    __syncthreads();
    if (lane < k) {
      S[lane] = snew;
      BACK[t * k + lane] = bi;
    }
    __syncthreads();
  }
  if (lane == 0) {
    int j = 0;
    float best = S[0];
    for (int i = 1; i < k; ++i)
      if (S[i] > best) { best = S[i]; j = i; }
    if (p.score) p.score[b] = best;
    for (int t = P - 1; t >= 0; --t) {
      p.path[int64_t(b) * P + t] = j;
      p.drafts[int64_t(b) * P + t] = ids[t * k + j];
      j = BACK[t * k + j];
    }
  }
}

void launch_select(const SelectArgs& a, size_t lds_bytes, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.B), dim3(64), lds_bytes, s, a);
}

// grid = (nchunks, B * bs), block = 256: best (value, id) key of one chunk.
__global__ __launch_bounds__(256) void verify_partial_kernel(VerifyArgs p) {
  __shared__ uint64_t red[4];
  const int c = blockIdx.x, row = blockIdx.y;
  const int v0 = c * p.chunk;
  const int v1 = min(p.V, v0 + p.chunk);
  const float* z = p.logits + int64_t(row) * p.V;
  uint64_t best = 0ull;
  if ((p.V & 3) == 0) {
    const int a0 = v0 >> 2, a1 = v1 >> 2;  // chunk is a multiple of 4
    const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
    for (int i = a0 + threadIdx.x; i < a1; i += blockDim.x) {
      const f32x4 x = z4[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t kk = rank_key(x[e], uint32_t(4 * i + e));
        best = kk > best ? kk : best;
      }
    }
  } else {
    for (int i = v0 + threadIdx.x; i < v1; i += blockDim.x) {
      const uint64_t kk = rank_key(z[i], uint32_t(i));
      best = kk > best ? kk : best;
    }
  }
  best = wave_max_u64(best);
  if ((threadIdx.x & (WAVE - 1)) == 0) red[threadIdx.x / WAVE] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < int(blockDim.x / WAVE); ++w) best = red[w] > best ? red[w] : best;
    best = red[0] > best ? red[0] : best;
    p.part[int64_t(row) * p.nchunks + c] = best;
  }
}

// One block per sequence: wave w merges the chunk keys of rows w, w + 4, ...;
// then one thread walks the rows to find the accepted prefix.
__global__ __launch_bounds__(256) void verify_final_kernel(VerifyArgs p) {
  extern __shared__ int32_t gl[];  // [bs] row argmaxes
  const int b = blockIdx.x;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  for (int i = wave; i < p.bs; i += blockDim.x / WAVE) {
    const uint64_t* part = p.part + int64_t(b * p.bs + i) * p.nchunks;
    uint64_t best = 0ull;
    for (int c = lane; c < p.nchunks; c += WAVE) best = part[c] > best ? part[c] : best;
    best = wave_max_u64(best);
    if (lane == 0) {
      const int g = best == 0ull ? 0 : int(key_id(best));
      gl[i] = g;
      if (p.argmax) p.argmax[int64_t(b) * p.bs + i] = g;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int P = p.bs - 1;
    int n = 0;
    while (n < P && gl[n] == p.drafts[int64_t(b) * P + n]) ++n;
    p.accepted[b] = n;
    p.bonus[b] = gl[n];
  }
}

void launch_verify_partial(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(verify_partial_kernel, dim3(a.nchunks, a.B * a.bs), dim3(256), 0, s, a);
}

void launch_verify_final(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(verify_final_kernel, dim3(a.B), dim3(256), size_t(a.bs) * 4, s, a);
}

}  // namespace dfl

// Training-side forward losses of the draft (NeMo AutoModel page,
// "Objective"): the position-decayed block cross-entropy over slots
// 1..bs-1, the selector cross-entropy over each position's top-k candidates
// scored against the ground-truth predecessor, and candidate_recall.
//
//   loss_rows_kernel  grid (B*(bs-1), chunks): per vocabulary chunk of a row,
//                     the running maximum and sum of exp of the transformed
//                     logits (one pass, online rescaling);
//   loss_seq_kernel   one block per sequence: merges a row's chunks in order
//                     into logsumexp, the label's CE, the candidate test and
//                     the selector CE (one wave per position, lane j =
//                     candidate j; pair scores in the lattice's float32
//                     order), and the sequence's partial sums;
//   loss_final_kernel one block: sums the sequences in order (double).
// This file is compiled with -ffp-contract=off so the pair scores round
// every product before adding it, as the selector does.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace dfl {

namespace {

__device__ __forceinline__ float loss_transform(float x, float mult, float cap) {
  float y = mult * x;
  if (cap > 0.0f) y = cap * tanhf(y / cap);
  return y;
}

// (m, s) <- merge of two (max, sum of exp(x - max)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * expf(m - m2) + s2;
    m = m2;
  } else if (m2 > -INFINITY) {
    s = s + s2 * expf(m2 - m);
  }
}

__device__ __forceinline__ void wave_lse(float& m, float& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, WAVE), s2 = __shfl_xor(s, o, WAVE);
    // both lanes of a pair must reach the same result: order the operands
    const bool mine_first = (threadIdx.x & o) == 0;
    float ma = mine_first ? m : m2, sa = mine_first ? s : s2;
    const float mb = mine_first ? m2 : m, sb = mine_first ? s2 : s;
    lse_merge(ma, sa, mb, sb);
    m = ma;
    s = sa;
  }
}

}  // namespace

// grid = (rows, nchunks), block = 256.
__global__ __launch_bounds__(256) void loss_rows_kernel(LossArgs p) {
  __shared__ float sm[8], ss[8];
  const int row = blockIdx.x, c = blockIdx.y;
  const int v0 = c * p.chunk, v1 = min(p.V, v0 + p.chunk);
  const float* z = p.logits + int64_t(row) * p.V;
  float m = -INFINITY, s = 0.0f;
  auto add = [&](float zv) {
    const float x = loss_transform(zv, p.mult, p.cap);
    if (x > m) {
      s = s * expf(m - x) + 1.0f;
      m = x;
    } else if (x > -INFINITY) {
      s += expf(x - m);
    }
  };
  if ((p.V & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0) {
    // chunks are multiples of 256 ids: non-temporal 16-byte loads, eight in
    // flight (a thread visits its values in the same order as with four)
    const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
    const int a0 = v0 >> 2, a1 = v1 >> 2;
    for (int i0 = a0 + threadIdx.x; i0 < a1; i0 += 8 * blockDim.x) {
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * blockDim.x;
        x[u] = i < a1 ? __builtin_nontemporal_load(z4 + i) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * int(blockDim.x) < a1) {
          add(x[u][0]); add(x[u][1]); add(x[u][2]); add(x[u][3]);
        }
    }
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += blockDim.x) add(z[v]);
  }
  wave_lse(m, s);
  const int w = threadIdx.x / WAVE;
  if ((threadIdx.x & (WAVE - 1)) == 0) { sm[w] = m; ss[w] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], S = ss[0];
    for (int i = 1; i < int(blockDim.x / WAVE); ++i) lse_merge(M, S, sm[i], ss[i]);
    p.part[(int64_t(row) * p.nchunks + c) * 2] = M;
    p.part[(int64_t(row) * p.nchunks + c) * 2 + 1] = S;
  }
}

// grid = B, block = 256 (4 waves; wave w takes positions w, w + 4, ...).
__global__ __launch_bounds__(256) void loss_seq_kernel(LossArgs p) {
  __shared__ double acc[4][4];   // per wave: sum w*CE, sum w, sum CE_sel, (unused)
  __shared__ int cnt[4][3];      // per wave: selector signals, supervised, hits
  const int b = blockIdx.x;
  const int wave = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const int P = p.P, k = p.k, r = p.r, V = p.V;
  double a_num = 0.0, a_den = 0.0, a_sel = 0.0;
  int n_sel = 0, n_sup = 0, n_hit = 0;
  for (int t = wave; t < P; t += 4) {
    const int64_t row = int64_t(b) * P + t;
    // logsumexp: the row's chunk partials, merged lane-wise then across lanes
    float m = -INFINITY, s = 0.0f;
    for (int c = lane; c < p.nchunks; c += WAVE)
      lse_merge(m, s, p.part[(row * p.nchunks + c) * 2], p.part[(row * p.nchunks + c) * 2 + 1]);
    wave_lse(m, s);
    const float lse = m + logf(s);
    const int lab = p.labels[row];
    const bool sup = lab >= 0 && lab < V;
    float ce = NAN, sce = NAN;
    bool hit = false;
    if (sup) {
      ce = lse - loss_transform(p.logits[row * V + lab], p.mult, p.cap);
      const int cj = lane < k ? p.ids[row * k + lane] : -1;
      const unsigned long long hits = __ballot(lane < k && cj == lab);
      hit = hits != 0ull;
      const int prev = t == 0 ? p.anchors[b] : p.labels[row - 1];
      if (hit && prev >= 0 && prev < V) {
        // s_j = pi(prev, c_j) + z_j in the selector's float32 order
        float sj = -INFINITY;
        if (lane < k) {
          const bool okc = cj >= 0 && cj < V;
          const float* ta = p.tl + int64_t(prev) * r;
          const float* tb = p.tr + int64_t(okc ? cj : 0) * r;
          float accp = 0.0f;
          int q = 0;
          if ((r & 3) == 0 && ((reinterpret_cast<uintptr_t>(p.tl) | reinterpret_cast<uintptr_t>(p.tr)) & 15) == 0) {
            for (; q + 16 <= r; q += 16) {
              f32x4 a4[4], c4[4];
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                a4[u] = *reinterpret_cast<const f32x4*>(ta + q + 4 * u);
                c4[u] = okc ? *reinterpret_cast<const f32x4*>(tb + q + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
              }
#pragma unroll
              for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const float prod = a4[u][e] * c4[u][e];
                  accp = accp + prod;
                }
            }
          }
          for (; q < r; ++q) {
            const float prod = ta[q] * (okc ? tb[q] : 0.0f);
            accp = accp + prod;
          }
          sj = accp + p.vals[row * k + lane];
        }
        const float mx = wave_max(sj);
        const float den = wave_sum(lane < k ? expf(sj - mx) : 0.0f);
        const int jt = __ffsll(static_cast<long long>(hits)) - 1;
        const float strue = __shfl(sj, jt, WAVE);
        sce = mx + logf(den) - strue;
      }
    }
    if (lane == 0) {
      if (p.block_ce) p.block_ce[row] = ce;
      if (p.selector_ce) p.selector_ce[row] = sce;
      if (sup) {
        const double wk = exp(-double(t) / double(p.gamma));
        a_num += wk * double(ce);
        a_den += wk;
        ++n_sup;
        if (hit) ++n_hit;
        if (!(sce != sce)) { a_sel += double(sce); ++n_sel; }
      }
    }
  }
  if (lane == 0) {
    acc[wave][0] = a_num; acc[wave][1] = a_den; acc[wave][2] = a_sel;
    cnt[wave][0] = n_sel; cnt[wave][1] = n_sup; cnt[wave][2] = n_hit;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double* o = p.seq + int64_t(b) * 6;
    double x0 = 0, x1 = 0, x2 = 0, c0 = 0, c1 = 0, c2 = 0;
    for (int w = 0; w < 4; ++w) {
      x0 += acc[w][0]; x1 += acc[w][1]; x2 += acc[w][2];
      c0 += cnt[w][0]; c1 += cnt[w][1]; c2 += cnt[w][2];
    }
    o[0] = x0; o[1] = x1; o[2] = x2; o[3] = c0; o[4] = c1; o[5] = c2;
  }
}

// One block of 64: sequences summed in order.
__global__ __launch_bounds__(64) void loss_final_kernel(LossArgs p) {
  if (threadIdx.x != 0) return;
  double x[6] = {0, 0, 0, 0, 0, 0};
  for (int b = 0; b < p.B; ++b)
    for (int i = 0; i < 6; ++i) x[i] += p.seq[int64_t(b) * 6 + i];
  const double block = x[1] > 0 ? x[0] / x[1] : 0.0;
  const double sel = x[3] > 0 ? x[2] / x[3] : 0.0;
  const double recall = x[4] > 0 ? x[5] / x[4] : 0.0;
  p.losses[0] = float(block + double(p.sel_weight) * sel);
  p.losses[1] = float(block);
  p.losses[2] = float(sel);
  p.losses[3] = float(recall);
}

void launch_loss_rows(const LossArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(loss_rows_kernel, dim3(a.B * a.P, a.nchunks), dim3(256), 0, s, a);
}

void launch_loss_seq(const LossArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(loss_seq_kernel, dim3(a.B), dim3(256), 0, s, a);
  hipLaunchKernelGGL(loss_final_kernel, dim3(1), dim3(64), 0, s, a);
}

}  // namespace dfl

// Path selector and greedy verification.
//
// Selector (NeMo AutoModel page, "Variants": a pairwise path selector walks
// one coherent path through each position's top-k candidates; "Objective":
// candidates are scored against the predecessor): one block per sequence.
// Per transition the factor-table rows of the previous and the current
// candidates are staged in LDS, all k*k pair scores are computed in
// float32 with separate multiply and add (m ascending), and a max-sum
// (Viterbi) step keeps the smallest predecessor on ties; the path is then
// traced back.  Only the listed order of float32 operations is used, so the
// result is bit-identical to any other evaluation in that order.
//
// Verification (NeMo SpeechLM page, "Validation"; llama-cpp-python wiki,
// "Prerequisites"): a row-wise argmax over the target logits, split into
// chunks so the whole logit tensor streams through HBM once, then a tiny
// kernel merges the chunks and finds the longest accepted prefix.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dfl {

// This file is compiled with -ffp-contract=off: every product below is
// rounded before it is added, and each pair's sum runs over m in order.
// Rows are padded to RS = r rounded up to 4 floats (+4) so they can be read
// 16 bytes at a time from LDS.
// Pairs (a0, b0), (a0, b1), (a1, b0), (a1, b1), accumulated side by side.
__device__ __forceinline__ void pair_dot2x2(const float* __restrict__ a0, const float* __restrict__ a1,
                                            const float* __restrict__ b0, const float* __restrict__ b1, int r,
                                            float (&out)[4]) {
  float c0 = 0.0f, c1 = 0.0f, c2 = 0.0f, c3 = 0.0f;
  int m = 0;
  for (; m + 4 <= r; m += 4) {
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(a0 + m), x1 = *reinterpret_cast<const f32x4*>(a1 + m);
    const f32x4 y0 = *reinterpret_cast<const f32x4*>(b0 + m), y1 = *reinterpret_cast<const f32x4*>(b1 + m);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = x0[e] * y0[e], p1 = x0[e] * y1[e], p2 = x1[e] * y0[e], p3 = x1[e] * y1[e];
      c0 = c0 + p0;
      c1 = c1 + p1;
      c2 = c2 + p2;
      c3 = c3 + p3;
    }
  }
  for (; m < r; ++m) {
    const float p0 = a0[m] * b0[m], p1 = a0[m] * b1[m], p2 = a1[m] * b0[m], p3 = a1[m] * b1[m];
    c0 = c0 + p0;
    c1 = c1 + p1;
    c2 = c2 + p2;
    c3 = c3 + p3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

__host__ __device__ int select_row_stride(int r) { return (r + 3) / 4 * 4 + 4; }

// 4-byte words of the selector's LDS (listed below), rounded up to even.
__host__ __device__ inline int select_lds_words(int k, int r, int P, int tw) {
  const int w = 2 * tw * k * select_row_stride(r) + tw * k * k + k + P * k + 2 * P + 3 * tw * k;
  return (w + 1) & ~1;
}

// One block of kSelThreads (1024) threads per sequence.  Pair scores depend
// only on the candidate ids, so a window of `tw` transitions is done at once:
// the table rows of its candidates are staged in LDS, all its pair scores are
// computed in parallel, then wave 0 runs the max-sum recursion over the
// window (lane j = candidate j, the scores S kept in registers; S in LDS
// carries them from one window to the next).
// LDS: TL [tw*k][RS], TR [tw*k][RS], PAIR [tw][k][k], S [k], BACK [P][k],
// PATH [P], TOK [2*tw*k], VAL [tw*k], CONF [P].
constexpr int kSelThreads = 1024;  // 16 waves: table gathers and pair scores in parallel

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs p, int tw) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = p.k, r = p.r, P = p.P, rs = select_row_stride(r);
  float* TL = lds;
  float* TR = TL + tw * k * rs;
  float* PAIR = TR + tw * k * rs;
  float* S = PAIR + tw * k * k;
  int32_t* BACK = reinterpret_cast<int32_t*>(S + k);
  int32_t* PATH = BACK + p.P * p.k;
  int32_t* TOK = PATH + p.P;
  float* VAL = reinterpret_cast<float*>(TOK + 2 * tw * p.k);
  const bool vec4 = (r & 3) == 0 &&
                    ((reinterpret_cast<uintptr_t>(p.tl) | reinterpret_cast<uintptr_t>(p.tr)) & 15) == 0;
  const int32_t* ids = p.ids + int64_t(b) * P * k;
  const float* vals = p.vals + int64_t(b) * P * k;
  const int V = p.V;
  const int anchor = p.anchors[b];
  if (p.cand) {
    // ---- fused candidate merge (at most 64 sorted lists per row): one wave
    // per row, lane l holding list l in registers; xor rounds over the lanes
    // each merge two lanes' lists into the 16 largest keys of both; after the
    // rounds d < max(lists, 16), lanes 0-15 hold the row's 16 best (keys are
    // unique), as the separate merge kernel finds them, and lane j < k
    // writes the j-th.  (The 16 shuffles of a round are independent; k
    // rounds of a wave maximum each, one shuffle after another, took ~15 us
    // longer at 7 rows of 19 lists.)
    const int wave = tid / WAVE, lane = tid & (WAVE - 1);
    const int nlists = p.count / p.glen;
    for (int t = wave; t < P; t += kSelThreads / WAVE) {
      const uint64_t* c = p.cand + (int64_t(b) * P + t) * p.count;
      uint64_t L[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        L[j] = (lane < nlists && j < p.glen) ? c[int64_t(lane) * p.lstride + int64_t(j) * p.kstride] : 0ull;
      for (int d = 1; d < max(nlists, 16); d <<= 1) {
        uint64_t brev[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) brev[j] = __shfl_xor(L[15 - j], d, WAVE);
        bitonic_top<16>(L, brev);
      }
      uint64_t best = L[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) best = lane == j ? L[j] : best;
      if (lane < k) {
        float z = p.multiplier * key_val(best);
        if (p.softcap > 0.f) z = p.softcap * tanhf(z / p.softcap);
        p.ids_out[(int64_t(b) * P + t) * k + lane] = int32_t(key_id(best));
        p.vals_out[(int64_t(b) * P + t) * k + lane] = z;
      }
    }
    __syncthreads();
  }

  for (int t0 = 0; t0 < P; t0 += tw) {
    const int nt = min(tw, P - t0);
    // ---- stage: the window's candidate ids (left rows: the previous
    // position's candidates, the anchor alone at t = 0; right rows: the
    // current position's), then their table rows, all loads of a thread
    // issued before any is used
    const int nrows = 2 * nt * k;
    for (int q = tid; q < nrows; q += kSelThreads) {
      const bool right = q >= nt * k;
      const int rr = right ? q - nt * k : q;
      const int w = rr / k, i = rr - w * k, t = t0 + w;
      int tok;
      if (right) tok = ids[t * k + i];
      else tok = t == 0 ? (i == 0 ? anchor : -1) : ids[(t - 1) * k + i];
      TOK[q] = (tok >= 0 && tok < V) ? tok : -1;
    }
    for (int q = tid; q < nt * k; q += kSelThreads) VAL[q] = vals[t0 * k + q];
    __syncthreads();
    if (vec4) {
      const int nv = r >> 2, total = nrows * nv;
      for (int e0 = 0; e0 < total; e0 += 16 * kSelThreads) {
        f32x4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + u * kSelThreads + tid;
          const int row = e / nv, mv = e - row * nv;
          const int tok = e < total ? TOK[row] : -1;
          const float* table = row >= nt * k ? p.tr : p.tl;
          v[u] = tok >= 0 ? *reinterpret_cast<const f32x4*>(table + int64_t(tok) * r + 4 * mv)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int e = e0 + u * kSelThreads + tid;
          const int row = e / nv, mv = e - row * nv;
          if (e < total) {
            float* dst = row >= nt * k ? TR + (row - nt * k) * rs : TL + row * rs;
            *reinterpret_cast<f32x4*>(dst + 4 * mv) = v[u];
          }
        }
      }
    } else {
      const int total = nrows * r;
      for (int e0 = 0; e0 < total; e0 += 8 * kSelThreads) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + u * kSelThreads + tid;
          const int row = e / r, m = e - row * r;
          const int tok = e < total ? TOK[row] : -1;
          const float* table = row >= nt * k ? p.tr : p.tl;
          v[u] = tok >= 0 ? table[int64_t(tok) * r + m] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int e = e0 + u * kSelThreads + tid;
          const int row = e / r, m = e - row * r;
          if (e < total) {
            float* dst = row >= nt * k ? TR + (row - nt * k) * rs : TL + row * rs;
            dst[m] = v[u];
          }
        }
      }
    }
    __syncthreads();
    // ---- pair scores of the window: PAIR[w][i][j] = pi(prev_i, cur_j).  A
    // thread takes a 2 x 2 block (rows i0, i0 + 1 against columns j0, j0 + 1)
    // so each staged row read from LDS feeds two chains.
    const int kh = (k + 1) >> 1;
    const int nblk = nt * kh * kh;
    for (int q = tid; q < nblk; q += kSelThreads) {
      const int w = q / (kh * kh), ij = q - w * kh * kh;
      const int i0 = 2 * (ij / kh), j0 = 2 * (ij - (ij / kh) * kh);
      const int i1 = min(i0 + 1, k - 1), j1 = min(j0 + 1, k - 1);
      const float* a0 = TL + (w * k + i0) * rs;
      const float* a1 = TL + (w * k + i1) * rs;
      const float* b0 = TR + (w * k + j0) * rs;
      const float* b1 = TR + (w * k + j1) * rs;
      float out[4];
      pair_dot2x2(a0, a1, b0, b1, r, out);
      float* dst = PAIR + w * k * k;
      dst[i0 * k + j0] = out[0];
      if (j0 + 1 < k) dst[i0 * k + j0 + 1] = out[1];
      if (i0 + 1 < k) dst[(i0 + 1) * k + j0] = out[2];
      if (i0 + 1 < k && j0 + 1 < k) dst[(i0 + 1) * k + j0 + 1] = out[3];
    }
    __syncthreads();
    if (p.debug_pair) {
      const int npairs = nt * k * k;
      for (int q = tid; q < npairs; q += kSelThreads) {
        const int w = q / (k * k), ij = q - w * k * k, i = ij / k, j = ij - i * k;
        const int t = t0 + w;
        p.debug_pair[(int64_t(b) * P + t) * k * k + ij] = PAIR[w * k * k + (t == 0 ? 0 : i) * k + j];
      }
    }
    // ---- max-sum recursion over the window (wave 0, lane j = candidate j).
    // The previous scores stay in registers and are broadcast with readlane;
    // every lane runs the same loads (lanes past k read candidate k - 1 and
    // store nothing), so the loop has no divergent branches.
    if (tid < WAVE) {
      const int j = tid, jj = min(j, k - 1);
      float s_cur = t0 > 0 ? S[jj] : 0.f;  // scores carried from the previous window
      for (int w = 0; w < nt; ++w) {
        const int t = t0 + w;
        const float* pr = PAIR + w * k * k;
        float snew;
        int bi = 0;
        if (t == 0) {
          snew = pr[jj] + VAL[jj];
        } else {
          float bv = 0.f;
          for (int i0 = 0; i0 < k; i0 += 16) {  // 16 column entries per LDS round trip
            float pv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) pv[u] = pr[min(i0 + u, k - 1) * k + jj];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const int i = i0 + u;
              const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_cur), min(i, k - 1))) + pv[u];
              if (i == 0) bv = v;
              else if ((i < k) & (v > bv)) { bv = v; bi = i; }
            }
          }
          snew = bv + VAL[w * k + jj];
        }
        s_cur = snew;
        if (j < k) BACK[t * k + j] = bi;
      }
      if (j < k) S[j] = s_cur;
    }
    __syncthreads();
  }
  // ---- trace back through LDS, then write the path and its tokens in parallel
  if (tid == 0) {
    int j = 0;
    float best = S[0];
    for (int i = 1; i < k; ++i)
      if (S[i] > best) { best = S[i]; j = i; }
    if (p.score) p.score[b] = best;
    for (int t = P - 1; t >= 0; --t) {
      PATH[t] = j;
      j = BACK[t * k + j];
    }
  }
  __syncthreads();
  for (int t = tid; t < P; t += kSelThreads) {
    const int j = PATH[t];
    p.path[int64_t(b) * P + t] = j;
    p.drafts[int64_t(b) * P + t] = ids[t * k + j];
  }
  if (!p.lens && !p.conf) return;
  // ---- confidence of each transition the path takes (llama-cpp-python
  // wiki, "Configuration Notes": draft_p_min stops a path before a
  // low-confidence selector transition): softmax over the k candidates of
  // the lattice's own float32 scores pi(c_prev, c_j) + z_j, c_prev = the
  // predecessor the path took.  One wave per position, lane j = candidate j;
  // pi is summed in the selector's order (multiply, then add, m ascending).
  float* CONF = VAL + tw * k;  // [P]
  const int wave = tid / WAVE, lane = tid & (WAVE - 1);
  for (int t = wave; t < P; t += kSelThreads / WAVE) {
    const int prev = t == 0 ? anchor : ids[(t - 1) * k + PATH[t - 1]];
    float sj = -INFINITY;
    if (lane < k) {
      const int cj = ids[t * k + lane];
      const bool okp = prev >= 0 && prev < V, okc = cj >= 0 && cj < V;
      const float* ta = p.tl + int64_t(okp ? prev : 0) * r;
      const float* tb = p.tr + int64_t(okc ? cj : 0) * r;
      float acc = 0.0f;
      int m = 0;
      if (vec4) {
        for (; m + 16 <= r; m += 16) {
          f32x4 a4[4], c4[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            a4[u] = okp ? *reinterpret_cast<const f32x4*>(ta + m + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
            c4[u] = okc ? *reinterpret_cast<const f32x4*>(tb + m + 4 * u) : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float prod = a4[u][e] * c4[u][e];
              acc = acc + prod;
            }
        }
      }
      for (; m < r; ++m) {
        const float a = okp ? ta[m] : 0.0f;
        const float c = okc ? tb[m] : 0.0f;
        const float prod = a * c;
        acc = acc + prod;
      }
      sj = acc + vals[t * k + lane];
    }
    const float mx = wave_max(sj);
    const float e = lane < k ? expf(sj - mx) : 0.0f;
    const float den = wave_sum(e);
    const float mine = __shfl(e, PATH[t], WAVE);
    if (lane == 0) {
      const float cf = mine / den;
      CONF[t] = cf;
      if (p.conf) p.conf[int64_t(b) * P + t] = cf;
    }
  }
  __syncthreads();
  if (p.lens && tid == 0) {
    const int hi = min(max(p.n_max, 0), P);
    const int lo = min(max(p.n_min, 0), hi);
    int n = P;
    for (int t = lo; t < P; ++t)
      if (CONF[t] < p.p_min) { n = t; break; }
    p.lens[b] = min(n, hi);
  }
}

// Transitions per window that fit the LDS budget (0: does not fit).
int select_window(int k, int r, int P, size_t budget) {
  const size_t per = size_t(2 * k * select_row_stride(r) + k * k + 3 * k) * 4;
  const size_t fixed = size_t(k + P * k + 2 * P) * 4;
  if (fixed + per > budget) return 0;
  return int(std::min<size_t>(size_t(P), (budget - fixed) / per));
}

static size_t select_lds_bytes(int k, int r, int P, int tw) { return size_t(select_lds_words(k, r, P, tw)) * 4; }

void launch_select(const SelectArgs& a, int tw, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.B), dim3(kSelThreads), select_lds_bytes(a.k, a.r, a.P, tw),
                     s, a, tw);
}

// grid = (nchunks, B * bs), block = 256: best (value, id) key of one chunk.
__global__ __launch_bounds__(256) void verify_partial_kernel(VerifyArgs p) {
  __shared__ uint64_t red[4];
  const int row = blockIdx.x, c = blockIdx.y;
  const int v0 = c * p.chunk;
  const int v1 = min(p.V, v0 + p.chunk);
  const float* z = p.logits + int64_t(row) * p.V;
  uint64_t best = 0ull;
  if ((p.V & 3) == 0) {
    const int a0 = v0 >> 2, a1 = v1 >> 2;  // chunk is a multiple of 4
    const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
    const int nt = blockDim.x;
    int i = a0 + threadIdx.x;
    // eight non-temporal 16-byte loads in flight per thread (four: fp8
    // high-batch scan 210 against 203 us, batched 46 against 43 us)
    for (; i + 7 * nt < a1; i += 8 * nt) {
      f32x4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = __builtin_nontemporal_load(z4 + i + u * nt);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint64_t kk = rank_key(x[u][e], uint32_t(4 * (i + u * nt) + e));
          best = kk > best ? kk : best;
        }
    }
    for (; i < a1; i += nt) {
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
  const int P = p.bs - 1;
  const int len = p.lens ? min(max(p.lens[b], 0), P) : P;
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < len && gl[n] == p.drafts[int64_t(b) * P + n]) ++n;
    p.accepted[b] = n;
    p.bonus[b] = gl[n];
  }
  if (p.draft_prob)
    for (int i = threadIdx.x; i < P; i += blockDim.x)
      p.draft_prob[int64_t(b) * P + i] = (i < len && gl[i] == p.drafts[int64_t(b) * P + i]) ? 1.0f : 0.0f;
}

void launch_verify_partial(const VerifyArgs& a, hipStream_t s) {
  // rows on x (up to 2^31 - 1 blocks), vocabulary chunks (at most 2048) on y
  hipLaunchKernelGGL(verify_partial_kernel, dim3(a.B * a.bs, a.nchunks), dim3(256), 0, s, a);
}

void launch_verify_final(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(verify_final_kernel, dim3(a.B), dim3(256), size_t(a.bs) * 4, s, a);
}

}  // namespace dfl

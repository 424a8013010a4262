// Compute-bound GEMMs y = x * W^T for many activation rows (batched drafts):
// the linears of the batched and fp8 high-batch workloads, where every
// weight row meets hundreds of activation rows and the matrix cores, not
// HBM, set the pace.
//
// Main loop: the DMA tile of dma_tile.h (256 weight rows x BM activation
// rows per block, both operands loaded straight into LDS).  Tile shapes:
//  * BM = 256, one block per CU (256 accumulators per lane), three stage
//    buffers for fp8 weights and two for bf16 (LDS);
//  * BM = 192 (fp8 weights): one block per CU, three stage buffers; a row
//    count that is a multiple of 192 but not of 256, or a tile count just
//    above a multiple of 256, wastes less;
//  * BM = 128 for at most 128 rows: fp8 two blocks per CU with two stage
//    buffers each, bf16 one block with three.
// Tiles are numbered with the activation tile fastest and dealt out so that
// each XCD (blocks go to the 8 XCDs round-robin) runs a contiguous run of
// tile numbers: the blocks that share a weight tile share that XCD's L2.
//
// Epilogues: float32 split-K partial sums (the same layout the
// weight-streaming kernels write, reduced by the consumer kernel), or with
// one K split the consumer itself, lane-local in both cases:
//  * SwiGLU: tile rows 0-63 and 128-191 are gate rows, rows 64-127 and
//    192-255 the matching up rows, so a lane holds gate and up of the same
//    column (acc[i] and acc[i + 2]);
//  * QKV: a tile's 256 rows are whole heads (d = 64 or 128) and the RoPE
//    partners (c, c + d/2) of a lane sit in acc[i] and acc[i + 2] (d = 128)
//    or acc[i] and acc[i + 1] (d = 64); q heads go to q_out, k and v heads
//    to this layer's cache rows.
// The lm_head of many rows has its own kernel (lmhead_tiled.hip).
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "common.h"
#include "dma_tile.h"
#include "kernels.h"

namespace dfl {

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
  GemmEpi epi;                                // consumer applied in the epilogue (one K split)
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

// Lane (r, h) of wave (wv, wm) holds, in acc[i][j][4 q + e], tile row
// 128 wv + 32 i + 8 q + 4 h + e (weight row per the tile's row map) of
// activation row m0 + BM/2 wm + 32 j + r.
template <typename TW, int BM, int R, int EPI, int OCC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OCC, OCC))) void gemm_tiled_kernel(TiledArgs p) {
  typedef DmaTile<TW, BM, R> T;
  constexpr int FJ = T::FJ, WM = T::WM;
  __shared__ __attribute__((aligned(1024))) char w0[T::WBYTES];
  __shared__ __attribute__((aligned(1024))) char w1[T::WBYTES];
  __shared__ __attribute__((aligned(1024))) char w2[R == 3 ? T::WBYTES : 16];
  __shared__ __attribute__((aligned(1024))) char x0[T::XBYTES];
  __shared__ __attribute__((aligned(1024))) char x1[T::XBYTES];
  __shared__ __attribute__((aligned(1024))) char x2[R == 3 ? T::XBYTES : 16];
  __shared__ float inv[BM];
  __shared__ double inv_freq[EPI == EPI_QKV ? 64 : 1];
  int mt, nt, split, group;
  if (!tiled_tile(p, mt, nt, split, group)) return;
  const int Mact = p.M_dev ? min(*p.M_dev, p.M) : p.M;
  const int m0 = mt * BM;
  if (m0 >= Mact) return;
  const int tid = threadIdx.x, lane = tid & (WAVE - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 1, wm = wave >> 1;
  const int r = lane & 31, h = lane >> 5;
  // first weight row of the 64 tile rows this wave loads
  const int F = p.epi.F;
  const int nw = EPI == EPI_SWIGLU ? (wave & 1 ? F : 0) + 128 * nt + 64 * (wave >> 1) : 256 * nt + 64 * wave;
  const TW* W = static_cast<const TW*>(p.groups > 1 ? p.Wg[group] : p.W);
  const float* scale = p.groups > 1 ? p.Sg[group] : p.scale;
  const int kb = split * p.k_split;
  const int nk = (min(p.K, kb + p.k_split) - kb) / kDmaKT;
  for (int t = tid; t < BM; t += blockDim.x) {
    float v = 1.f;
    const int m = m0 + t;
    if (p.rs.sumsq && m < Mact) {
      const float s = sum_in_order(p.rs.sumsq + int64_t(m) * p.rs.blocks, p.rs.blocks);
      v = 1.0f / sqrtf(s * p.rs.inv_width + p.rs.eps);
    }
    inv[t] = v;
  }
  if (EPI == EPI_QKV && tid < p.epi.d / 2)
    inv_freq[tid] = pow(double(p.epi.theta), -2.0 * double(tid) / double(p.epi.d));
  f32x16 acc[4][FJ];
  T::run(p.X, p.ldx, W, p.ldw, p.N, Mact, nw, m0, kb, nk, wave, w0, w1, w2, x0, x1, x2, acc);
  __syncthreads();  // inv and inv_freq visible
  // weight row of (i, q, h) (element e adds e)
  auto wrow = [&](int i, int q) {
    if (EPI == EPI_SWIGLU) return ((i >> 1) ? F : 0) + 128 * nt + 64 * wv + 32 * (i & 1) + 8 * q + 4 * h;
    return 256 * nt + 128 * wv + 32 * i + 8 * q + 4 * h;
  };
  // scale to the stored value: per weight row (fp8) and per activation row (RMSNorm)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nb = wrow(i, q);
      float s[4] = {1.f, 1.f, 1.f, 1.f};
      if (scale) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = scale[min(nb + e, p.N - 1)];
      }
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const float iv = inv[WM * wm + 32 * j + r];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = (acc[i][j][4 * q + e] * s[e]) * iv;
      }
    }
  }
  if (EPI == EPI_NONE) {
    float* P = p.P + int64_t(group) * p.group_stride + int64_t(split) * p.split_stride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nb = wrow(i, q);
        if (nb >= p.N) continue;
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          const int m = m0 + WM * wm + 32 * j + r;
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
  if (EPI == EPI_SWIGLU) {
    bf16_t* out = static_cast<bf16_t*>(p.epi.act_out);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f = wrow(i, q);
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
          const int m = m0 + WM * wm + 32 * j + r;
          if (m >= Mact) continue;
          uint32_t o[2];
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            float y[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float gt = acc[i][j][4 * q + e + u];
              const float up = acc[i + 2][j][4 * q + e + u];
              // hardware exponential (a few float ulp; the outputs are bf16):
              // 621 -> 605 us for the fp8 high-batch gate/up projection
              y[u] = gt / (1.0f + __expf(-gt)) * up;
            }
            o[e / 2] = f32x2_to_bf16x2(y[0], y[1]);
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
  // EPI_QKV: element (i, q, e) with column c < d/2 of its head pairs with c + d/2
  const GemmEpi& e = p.epi;
  const int d = e.d, half = d / 2, nh = e.nq + 2 * e.nkv;
  bf16_t* qo = static_cast<bf16_t*>(e.q_out);
  bf16_t* kc = static_cast<bf16_t*>(e.k_layer);
  bf16_t* vc = static_cast<bf16_t*>(e.v_layer);
  // acc[I] holds columns c < d/2 of its head, acc[IP] the partners c + d/2
  auto emit = [&](auto Ic, auto IPc) {
    constexpr int i = decltype(Ic)::value, ip = decltype(IPc)::value;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c0 = wrow(i, q);                     // output column of the first element
      const int head = c0 / d, ci = c0 % d;          // ci < d/2
      if (head >= nh) continue;
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int m = m0 + WM * wm + 32 * j + r;
        if (m >= Mact) continue;
        const int b = m / e.bs, t = m % e.bs;
        const int pos = e.ctx_lens[b] + t;
        float y0[4], y1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float xa = acc[i][j][4 * q + u];
          const float xb = acc[ip][j][4 * q + u];
          if (head < e.nq + e.nkv) {
            // angle in double, reduced to [-pi, pi], then the hardware sine
            // and cosine (~1e-6 absolute error there, far below the bf16
            // outputs' rounding; the library sincosf made the fp8 high-batch
            // QKV projection 170 against 159 us)
            const double ang = double(pos) * inv_freq[ci + u];
            const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
            float sn, cs;
            __sincosf(float(red), &sn, &cs);
            y0[u] = xa * cs - xb * sn;
            y1[u] = xb * cs + xa * sn;
          } else {
            y0[u] = xa;
            y1[u] = xb;
          }
        }
        const u32x2 lo = {f32x2_to_bf16x2(y0[0], y0[1]),
                          f32x2_to_bf16x2(y0[2], y0[3])};
        const u32x2 hi = {f32x2_to_bf16x2(y1[0], y1[1]),
                          f32x2_to_bf16x2(y1[2], y1[3])};
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
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if (d == 128) {
    emit(I0{}, I2{});
    emit(I1{}, I3{});
  } else {
    emit(I0{}, I1{});
    emit(I2{}, I3{});
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
TiledShape tiled_shape(int weight_dtype, int M, int bm) {
  if (bm != 128 && bm != 256 && !(bm == 192 && weight_dtype == 2)) bm = M > 128 ? 256 : 128;
  if (const char* env = std::getenv("DFLASH2_TILED_BM")) {
    const int v = std::atoi(env);
    if (v == 128 || v == 256 || (v == 192 && weight_dtype == 2)) bm = v;
  }
  // fp8 128-row tiles: two blocks per CU (two 32 KB stage buffers each)
  return TiledShape{bm, (bm == 128 && weight_dtype == 2) ? 2 : 1};
}

bool gemm_tiled_ok(int weight_dtype, int M, int K) {
  return weight_dtype != 0 && M > kTiledMinRowsGemm && K % kDmaKT == 0;
}

template <typename TW, int BM, int R, int OCC>
static void launch_tiled_t(const TiledArgs& t, hipStream_t s) {
  const dim3 grid(unsigned((t.tiles + 7) / 8 * 8));
  if (t.epi.kind == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_tiled_kernel<TW, BM, R, EPI_SWIGLU, OCC>), grid, dim3(256), 0, s, t);
  else if (t.epi.kind == EPI_QKV)
    hipLaunchKernelGGL((gemm_tiled_kernel<TW, BM, R, EPI_QKV, OCC>), grid, dim3(256), 0, s, t);
  else hipLaunchKernelGGL((gemm_tiled_kernel<TW, BM, R, EPI_NONE, OCC>), grid, dim3(256), 0, s, t);
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
  const TiledShape sh = tiled_shape(weight_dtype, a.M, a.tile_rows);
  t.nM = (a.M + sh.bm - 1) / sh.bm;
  t.nN = t.epi.kind == EPI_SWIGLU ? (a.epi.F + 127) / 128 : (a.N + kDmaBN - 1) / kDmaBN;
  t.tiles = t.nM * t.nN * t.splits * t.groups;
  if (weight_dtype == 1) {
    if (sh.bm == 256) launch_tiled_t<bf16_t, 256, 2, 1>(t, s);
    else launch_tiled_t<bf16_t, 128, 3, 1>(t, s);
  } else {
    if (sh.bm == 256) launch_tiled_t<fp8_t, 256, 3, 1>(t, s);
    else if (sh.bm == 192) launch_tiled_t<fp8_t, 192, 3, 1>(t, s);
    else launch_tiled_t<fp8_t, 128, 2, 2>(t, s);
  }
}

}  // namespace dfl

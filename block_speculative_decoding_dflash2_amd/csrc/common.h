// Device helpers shared by the gfx950 kernels: storage types, conversions,
// the 16x16x32 MFMA step, wave reductions and the ranking key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef uint8_t fp8_t;    // OCP e4m3fn code

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x1 __attribute__((ext_vector_type(1)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two floats to two bf16 (low half: lo), rounded to nearest even by the
// hardware conversion (one instruction per pair; the same bits as adding
// 0x7FFF plus the kept lsb and truncating, for the finite inputs here).
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
  typedef float f32x2_hw __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_hw{lo, hi}, bf16x2_hw));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return bf16_t(f32x2_to_bf16x2(f, 0.f) & 0xFFFFu); }

template <typename T> struct Act;
template <> struct Act<float> {
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Act<bf16_t> {
  __device__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---------------------------------------------------------------------------
// One MFMA "k32 step": D[16 x 16] += A[16 x 32] * B[32 x 16].
// Lane l supplies row (l % 16) of A and column (l % 16) of B, and the eight
// contraction indices of its lane group g = l / 16.  Which physical k each of
// the eight slots (g, j) stands for is the caller's choice, as long as A and
// B agree.  Output: lane l holds D[4 * (l / 16) + i][l % 16], i = 0..3.
// ---------------------------------------------------------------------------
struct Frag8Bf16 { bf16x8 v; };
struct Frag8F32 { float v[8]; };

__device__ __forceinline__ f32x4 mfma_k32(const Frag8Bf16& a, const Frag8Bf16& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k32(const Frag8F32& a, const Frag8F32& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// Eight consecutive elements of a row, loaded as an MFMA fragment.
template <typename T> struct FragOf;
template <> struct FragOf<bf16_t> { typedef Frag8Bf16 type; };
template <> struct FragOf<float> { typedef Frag8F32 type; };

__device__ __forceinline__ void load_frag(Frag8Bf16& f, const bf16_t* p) {
  u32x4 u = *reinterpret_cast<const u32x4*>(p);
  f.v = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void load_frag(Frag8F32& f, const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
}
__device__ __forceinline__ void zero_frag(Frag8Bf16& f) { f.v = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }
__device__ __forceinline__ void zero_frag(Frag8F32& f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
}

// Eight fp8 e4m3fn codes -> eight bf16 (exact: every e4m3 value is a bf16
// value).  gfx950 converts two codes straight to two bf16 per instruction
// (unit scale); checked on MI355X to give the same bits as widening to
// float32 and keeping the upper half, for all 256 codes.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp8x8_to_frag(Frag8Bf16& f, u32x2 codes) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(codes[0]), 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(codes[0]), 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(codes[1]), 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(codes[1]), 1.0f, true);
  const u32x4 u = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                   __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  f.v = __builtin_bit_cast(bf16x8, u);
}

// Weight fragment loaders by weight storage type.
template <typename TW> struct WFrag;
template <> struct WFrag<bf16_t> {
  typedef Frag8Bf16 frag;
  typedef u32x4 raw;
  __device__ static raw load(const bf16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
  __device__ static raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  }
  __device__ static void cvt(frag& f, raw r) { f.v = __builtin_bit_cast(bf16x8, r); }
};
template <> struct WFrag<fp8_t> {
  typedef Frag8Bf16 frag;
  typedef u32x2 raw;
  __device__ static raw load(const fp8_t* p) { return *reinterpret_cast<const u32x2*>(p); }
  __device__ static raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  }
  __device__ static void cvt(frag& f, raw r) { fp8x8_to_frag(f, r); }
};
struct RawF32x8 { f32x4 a, b; };
template <> struct WFrag<float> {
  typedef Frag8F32 frag;
  typedef RawF32x8 raw;
  __device__ static raw load(const float* p) {
    RawF32x8 r;
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
    return r;
  }
  __device__ static void cvt(frag& f, raw r) {
    f.v[0] = r.a[0]; f.v[1] = r.a[1]; f.v[2] = r.a[2]; f.v[3] = r.a[3];
    f.v[4] = r.b[0]; f.v[5] = r.b[1]; f.v[6] = r.b[2]; f.v[7] = r.b[3];
  }
};

// ---------------------------------------------------------------------------
// Wave / block reductions.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, WAVE);
    v = w > v ? w : v;
  }
  return v;
}

// Sum over a block of `nthreads` (multiple of 64, <= 1024); every thread gets
// the total.  `red` is LDS scratch of >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  __syncthreads();
  if ((threadIdx.x & (WAVE - 1)) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// ---------------------------------------------------------------------------
// Ranking key: (value desc, id asc) as one unsigned 64-bit integer whose
// natural order is the ranking order.  -0.0 is ranked as +0.0; NaN ranks
// below every number.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t ordered_f32(float v) {
  v = v + 0.0f;                                  // -0.0 -> +0.0
  uint32_t u = __float_as_uint(v);
  if (v != v) return 0u;                         // NaN: lowest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t rank_key(float v, uint32_t id) {
  return (uint64_t(ordered_f32(v)) << 32) | uint64_t(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - uint32_t(k); }

// a (KMAX keys, largest first) <- the KMAX largest keys of a and b, largest
// first, where brev holds b smallest first: max(a[i], brev[i]) is a bitonic
// sequence holding them, sorted by a half-cleaner cascade.
template <int KMAX>
__device__ __forceinline__ void bitonic_top(uint64_t (&a)[KMAX], const uint64_t (&brev)[KMAX]) {
#pragma unroll
  for (int i = 0; i < KMAX; ++i) a[i] = a[i] > brev[i] ? a[i] : brev[i];
#pragma unroll
  for (int half = KMAX / 2; half >= 1; half >>= 1) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if ((i & half) == 0) {
        const uint64_t x = a[i], y = a[i + half];
        a[i] = x > y ? x : y;
        a[i + half] = x > y ? y : x;
      }
    }
  }
}

__device__ __forceinline__ float key_val(uint64_t k) { return unordered_f32(uint32_t(k >> 32)); }

// Sum of p[0..n) added in index order, with the loads of 32 consecutive
// values issued together (one memory round trip per 32 values rather than
// one per value).  Used for an activation row's per-column-block sums of
// squares, from which a GEMM applies the row's RMSNorm factor.
__device__ __forceinline__ float sum_in_order(const float* __restrict__ p, int n) {
  float s = 0.f;
  for (int c = 0; c < n; c += 32) {
    float v[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = p[min(c + e, n - 1)];
#pragma unroll
    for (int e = 0; e < 32; ++e)
      if (c + e < n) s += v[e];
  }
  return s;
}

}  // namespace dfl

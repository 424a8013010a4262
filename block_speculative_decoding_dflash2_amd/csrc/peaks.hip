// Measured ceilings of this chip, for the roofline fractions the benchmark
// reports beside the nominal ones: the bf16 matrix-core rate on operands held
// in registers (no memory traffic at all), with random or all-zero operands
// (the rate depends on the data: random operands draw more power and the
// clock drops), and the HBM read rate of a plain streaming read.
#include "common.h"
#include "dflash2.h"

namespace dfl {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One wave per SIMD; each wave keeps 16 independent 32x32 accumulators, so
// consecutive MFMAs never wait for each other.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, int zero, float* out) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  // operand bits: a per-lane xorshift sequence, mapped to bf16 values in
  // [-2, 2) (exponent bits forced so no NaN or infinity occurs)
  uint32_t st = tid * 2654435761u + 12345u;
  auto next = [&]() {
    st ^= st << 13;
    st ^= st >> 17;
    st ^= st << 5;
    return st;
  };
  u32x4 ua[4], ub[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t ra = next(), rb = next();
      // bf16 = sign | exponent 126..127 | random mantissa, two per word
      const uint32_t ma = (ra & 0x807F807Fu) | 0x3F003F00u | ((ra >> 7) & 0x00800080u);
      const uint32_t mb = (rb & 0x807F807Fu) | 0x3F003F00u | ((rb >> 7) & 0x00800080u);
      ua[i][e] = zero ? 0u : ma;
      ub[i][e] = zero ? 0u : mb;
    }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ua[i]),
                                                            __builtin_bit_cast(bf16x8, ub[j]), acc[i][j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  if ((threadIdx.x & (WAVE - 1)) == 0) out[tid / WAVE] = s;
}

// Grid-stride read of n16 16-byte words with non-temporal loads, four in
// flight per thread; one partial sum per thread keeps the loads alive.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src, int64_t n16, uint32_t* out) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

}  // namespace dfl

extern "C" {

dflash2_status dflash2_peak_mfma(hipStream_t stream, int32_t blocks, int32_t iters, int32_t zero_operands,
                                 float* out) {
  if (blocks < 1 || iters < 1 || !out) return DFLASH2_ERR_INVALID_ARG;
  hipLaunchKernelGGL(dfl::peak_mfma_kernel, dim3(blocks), dim3(256), 0, stream, iters, zero_operands ? 1 : 0, out);
  return hipGetLastError() == hipSuccess ? DFLASH2_OK : DFLASH2_ERR_HIP;
}

dflash2_status dflash2_peak_read(hipStream_t stream, const void* src, size_t bytes, int32_t blocks,
                                 uint32_t* out) {
  if (!src || !out || blocks < 1 || bytes < 16 || (reinterpret_cast<uintptr_t>(src) & 15))
    return DFLASH2_ERR_INVALID_ARG;
  hipLaunchKernelGGL(dfl::peak_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const dfl::u32x4*>(src), int64_t(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? DFLASH2_OK : DFLASH2_ERR_HIP;
}

}  // extern "C"

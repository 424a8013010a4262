// A stand-in for the few HIP runtime entry points the library's host code
// calls, for the sanitized CPU build of that host code (no GPU, no HIP
// runtime): kernel launches are recorded and checked for sane launch shapes,
// events and device queries succeed, and the static scratch array's device
// address is a fixed fake value.  Test infrastructure only.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {
dim3 g_grid, g_block;
long g_launches = 0;
long g_bad = 0;
}  // namespace

extern "C" {

long hc_launches() { return g_launches; }
long hc_bad_launches() { return g_bad; }

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t, hipStream_t) {
  g_grid = grid;
  g_block = block;
  return hipSuccess;
}
hipError_t __hipPopCallConfiguration(dim3* grid, dim3* block, size_t* shm, hipStream_t* stream) {
  *grid = g_grid;
  *block = g_block;
  *shm = 0;
  *stream = nullptr;
  return hipSuccess;
}
void** __hipRegisterFatBinary(const void*) {
  static void* handle = nullptr;
  return &handle;
}
void __hipRegisterFunction(void**, const void*, char*, const char*, unsigned int, uint3*, uint3*, dim3*, dim3*, int*) {}
void __hipRegisterVar(void**, void*, char*, char*, int, size_t, int, int) {}
void __hipUnregisterFatBinary(void**) {}

hipError_t hipLaunchKernel(const void* f, dim3 grid, dim3 block, void** args, size_t shm, hipStream_t) {
  ++g_launches;
  const unsigned long long blocks = 1ull * grid.x * grid.y * grid.z;
  const unsigned threads = block.x * block.y * block.z;
  if (!f || !args || blocks == 0 || grid.x > 0x7FFFFFFFu || grid.y > 65535u || grid.z > 65535u || threads == 0 ||
      threads > 1024u || shm > 160 * 1024) {
    ++g_bad;
    std::fprintf(stderr, "bad launch: grid %u %u %u block %u %u %u shm %zu\n", grid.x, grid.y, grid.z, block.x,
                 block.y, block.z, shm);
  }
  return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** p, const void*) {
  *p = reinterpret_cast<void*>(uintptr_t(0x7000000000ull));
  return hipSuccess;
}

}  // extern "C"

// Small device utilities of the library's host sequencing: a fill kernel that
// the kernel timer uses to evict the caches (L2 and the MALL) before a timed
// launch.  No layer arithmetic lives here.
#include "cca_internal.h"

namespace cca {
namespace {

// Grid-stride 16-byte stores of one 32-bit pattern over n16 chunks.
__global__ __launch_bounds__(256) void fill_u32x4_kernel(uint4* p, long n16, uint32_t v) {
  const uint4 q = make_uint4(v, v, v, v);
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n16; i += (long)gridDim.x * 256) p[i] = q;
}

}  // namespace

hipError_t launch_fill(void* p, size_t bytes, uint32_t v, hipStream_t s) {
  if (((uintptr_t)p & 15u) != 0 || bytes % 16 != 0) return hipErrorInvalidValue;
  const long n16 = (long)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const long want = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fill_u32x4_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<uint4*>(p),
                     n16, v);
  return hipGetLastError();
}

}  // namespace cca

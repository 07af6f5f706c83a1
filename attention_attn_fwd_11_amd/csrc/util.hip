// util.hip -- small helper kernels for the ABI layer.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

// Zero-fills `n16` 16-byte words (a kernel rather than a memset so the call
// can sit inside a captured HIP graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t stream) {
  // Callers pass 16-byte aligned buffers whose size is a multiple of 16
  // bytes (rows of 64 or 128 features of 2 or 4 bytes).
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<u32x4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace attn

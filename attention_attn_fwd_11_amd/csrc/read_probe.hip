// read_probe.hip -- streaming-read bandwidth probe (measurement context only).
//
// Built as its own library (libattn_probe.so), not part of the attention C
// ABI.  One kernel reads a device buffer once with grid-stride 16-byte
// nontemporal loads (eight independent loads in flight per lane; the hint
// streams past cache retention, ~7 TB/s against ~6.2 TB/s for ordinary
// loads on an MI355X) and writes one word per thread,
// so the bytes moved are the buffer size plus a negligible 4 bytes per
// thread.  The benchmark times it beside the decode kernels to show what a
// plain streaming read achieves on the same device.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ p, size_t n16,
                                                    unsigned* __restrict__ out) {
  u32x4 acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// Words the probe writes for `blocks` workgroups (256 threads each).
size_t attn_probe_out_words(int32_t blocks) { return blocks > 0 ? (size_t)blocks * 256 : 0; }

// Reads `bytes` (a multiple of 16, 16-byte aligned) from `buf` once; writes
// attn_probe_out_words(blocks) unsigned words to `out`.  Returns 0, or 1 for
// invalid arguments, or 2 if the launch failed.  Enqueued on `stream`.
int attn_probe_stream_read(const void* buf, size_t bytes, void* out, int32_t blocks, void* stream) {
  if (!buf || !out || blocks <= 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15u)) return 1;
  hipLaunchKernelGGL(stream_read, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, static_cast<unsigned*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"

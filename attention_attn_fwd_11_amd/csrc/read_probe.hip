// read_probe.hip -- measurement-context probes (not part of the attention path).
//
// Built as its own library (libattn_probe.so), not part of the attention C
// ABI.  The benchmark times them beside the attention kernels to show what
// plain kernels achieve on the same device under the same sustained load.
//
//   stream_read  reads a device buffer once with grid-stride 16-byte
//                nontemporal loads (eight independent loads in flight per
//                lane; the hint streams past cache retention, ~7 TB/s against
//                ~6.2 TB/s for ordinary loads on an MI355X) and writes one
//                word per thread, so the bytes moved are the buffer size plus
//                a negligible 4 bytes per thread.
//   mfma_stream  issues nothing but v_mfma_f32_32x32x16_bf16 from registers:
//                eight waves per workgroup (two per SIMD, the prefill's
//                occupancy), one workgroup per compute unit, four independent
//                accumulators per wave, operands drawn from a random bf16
//                buffer so the matrix cores switch real data.  Its rate is
//                what the matrix cores sustain, at the clock the chip holds
//                under that load, when nothing else runs.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMfmaThreads = 512;
constexpr int kMfmaOperandSets = 4;
constexpr size_t kMfmaHoldLds = 96 * 1024;   // > half of the 160 KiB: one workgroup per CU

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

// ops: 2 * kMfmaOperandSets * 64 vectors of 8 bf16 (set s: A at 2s, B at
// 2s + 1, one vector per lane).  Per wave and iteration: 16 MFMAs.
__global__ __launch_bounds__(kMfmaThreads) void mfma_stream(const bf16x8* __restrict__ ops, int iters,
                                                           float* __restrict__ out) {
  extern __shared__ float hold[];
  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) hold[0] = 0.f;
  bf16x8 a[kMfmaOperandSets], b[kMfmaOperandSets];
#pragma unroll
  for (int s = 0; s < kMfmaOperandSets; ++s) {
    a[s] = ops[(2 * s) * 64 + lane];
    b[s] = ops[(2 * s + 1) * 64 + lane];
  }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k)
      acc[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k & 3], b[(k >> 2) & 3], acc[k & 3], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += acc[c][e];
  __syncthreads();
  out[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = sum + hold[0];
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

// Bytes of the operand buffer attn_probe_mfma reads (random bf16 values).
size_t attn_probe_mfma_operand_bytes() { return (size_t)2 * kMfmaOperandSets * 64 * 16; }

// Floating-point operations of one attn_probe_mfma launch.
double attn_probe_mfma_flops(int32_t blocks, int32_t iters) {
  return blocks > 0 && iters > 0 ? (double)blocks * (kMfmaThreads / 64) * iters * 16 * (2.0 * 32 * 32 * 16) : 0.0;
}

// Runs `blocks` workgroups (give the compute-unit count) of mfma_stream for
// `iters` iterations; reads attn_probe_mfma_operand_bytes() from `ops`
// (16-byte aligned) and writes blocks * 512 floats to `out`.  Returns 0, 1
// for invalid arguments, 2 if the launch failed.  Enqueued on `stream`.
int attn_probe_mfma(const void* ops, void* out, int32_t blocks, int32_t iters, void* stream) {
  if (!ops || !out || blocks <= 0 || iters <= 0 || (reinterpret_cast<uintptr_t>(ops) & 15u)) return 1;
  hipLaunchKernelGGL(mfma_stream, dim3((unsigned)blocks), dim3(kMfmaThreads), kMfmaHoldLds,
                     static_cast<hipStream_t>(stream), static_cast<const bf16x8*>(ops), iters,
                     static_cast<float*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"

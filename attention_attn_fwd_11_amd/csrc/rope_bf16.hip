// rope_bf16.hip -- the rotary position embedding applied to key rows once,
// into a separate buffer, ahead of the attention kernel.  "GPU learning day
// 24: Operator Fusion", section 6 (exercise 1's reference answer), places
// RoPE either in the epilogue of the QKV projection or inside the attention
// kernel; this pass stands in for the former for K, so each key is rotated
// once instead of once per query tile that reads it.  The arithmetic is the
// attention kernel's own (rope8), so both placements give identical bits.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

// One item = (key row, slot pair sl): the 8 features 8*sl .. 8*sl+7 and
// their partners at + d/2.  A workgroup takes 256 consecutive items of one
// head (blockIdx.x = head * tiles + tile), so both 16-byte loads and stores
// of a wave are contiguous and all indexing inside a head is 32-bit.  Bound
// by HBM: 4 bytes per element (read and write) plus table rows from L2.
template <int D>
__global__ __launch_bounds__(256) void rope_rows_kernel(const uint16_t* __restrict__ src,
                                                        uint16_t* __restrict__ dst,
                                                        const float* __restrict__ table,
                                                        const int32_t* __restrict__ kv_lens,
                                                        int H, int S, int tiles) {
  constexpr int HS = D / 16;
  const int bh = blockIdx.x / tiles;                       // b * H + h
  const int it = (blockIdx.x - bh * tiles) * 256 + threadIdx.x;
  const int j = it / HS, sl = it % HS;
  const int n = kv_lens ? min(max(kv_lens[bh / H], 0), S) : S;
  if (j >= n) return;                                      // never read by the attention kernel
  const int64_t off = ((int64_t)bh * S + j) * D + 8 * sl;
  u32x4 x1 = ld16(src + off), x2 = ld16(src + off + D / 2);
  const float* c = table + j * D + 8 * sl;
  rope8(x1, x2, *reinterpret_cast<const f32x4*>(c), *reinterpret_cast<const f32x4*>(c + 4),
        *reinterpret_cast<const f32x4*>(c + D / 2), *reinterpret_cast<const f32x4*>(c + D / 2 + 4));
  st16(dst + off, x1);
  st16(dst + off + D / 2, x2);
}

template <int D>
hipError_t launch_d(const void* src, void* dst, const float* table, const int32_t* kv_lens, int B,
                    int H, int S, hipStream_t stream) {
  const int64_t tiles = ((int64_t)S * (D / 16) + 255) / 256;   // per head
  const int64_t blocks = tiles * B * H;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_rows_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), table, kv_lens,
                     H, S, (int)tiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_rows(const void* src, void* dst, const float* table, const int32_t* kv_lens,
                            int B, int H, int S, int d, hipStream_t stream) {
  if (d == 64) return launch_d<64>(src, dst, table, kv_lens, B, H, S, stream);
  if (d == 256) return launch_d<256>(src, dst, table, kv_lens, B, H, S, stream);
  return launch_d<128>(src, dst, table, kv_lens, B, H, S, stream);
}

}  // namespace attn

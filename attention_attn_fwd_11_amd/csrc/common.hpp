// common.hpp -- small device helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Base-2 logarithm (v_log_f32).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// fp32 -> bf16 bits, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Two fp32 -> one dword of two bf16 (lo in bits 0..15), round to nearest
// even, in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// bf16 halves of a dword -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// (1.0, 1.0) in bf16: dot2 with it sums the two halves of a packed pair.
#define kOnesBf16x2 (as_bf16x2(0x3f803f80u))

// LDS transpose read (ds_read_b64_tr_b16).  Within each 16-lane group the
// four rows x sixteen columns of 16-bit elements addressed by the group are
// transposed: source lane s supplies the address of row s/4, columns
// 4*(s%4) .. 4*(s%4)+3 of the block, and result lane j receives column j of
// rows 0..3 (element e = row e).
__device__ __forceinline__ u32x2 lds_read_tr16x4(const void* lds_generic) {
  const lds_i16x4* p = (const lds_i16x4*)(const __attribute__((address_space(3))) void*)lds_generic;
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4*>(p));
  return __builtin_bit_cast(u32x2, r);
}

// LDS byte swizzle at 16-byte granularity for row-major tiles of 8..16
// 16-byte slots per row.  Row r's slot s is stored at slot s ^ sw(r) with
// sw(r) = 2*(r&3) | ((r>>2)&1) | (r&8).  Two access patterns are then free of
// bank conflicts: 8 consecutive rows reading the same slot (a permutation of
// slot%8 over the rows) and 4 consecutive rows (aligned to 4) reading the same
// even-aligned slot pair (the transpose reads: the pair index moves by r&3).
__device__ __forceinline__ int lds_swizzle(int row) {
  return ((row & 3) << 1) | ((row >> 2) & 1) | (row & 8);
}

// LDS-poison debug build (compiled with ATTN_LDS_POISON into
// libattn_lds_poison.so): before a direct copy lands lane i's 16 bytes at
// lds_base + 16*i, the lane writes bf16 NaNs there and waits for the write,
// so any read of a staging buffer that is not ordered after the copy's
// completion (a missing wait or barrier) returns NaN and fails parity instead
// of silently reading the previous tile.  A no-op in the normal build.
__device__ __forceinline__ void lds_poison_lane(void* lds_base) {
#ifdef ATTN_LDS_POISON
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  *reinterpret_cast<u32x4*>(static_cast<unsigned char*>(lds_base) + 16 * lane) =
      u32x4{0x7fc17fc1u, 0x7fc17fc1u, 0x7fc17fc1u, 0x7fc17fc1u};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
  (void)lds_base;
#endif
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane i's 16 bytes land at lds_base + 16*i; lds_base must be wave-uniform.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void global_to_lds16(const void* g, void* lds_base) {
  lds_poison_lane(lds_base);
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 0);
}

// Streaming forms of the 16-byte loads for data read exactly once (decode's
// K and V): the nontemporal hint ("nt") reaches ~7 TB/s on an MI355X against
// ~6.2 TB/s for ordinary loads in a streaming-read probe.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void global_to_lds16_stream(const void* g, void* lds_base) {
  lds_poison_lane(lds_base);
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_base, 16, 0, 2);   // cache policy 2: nt
}

// Buffer resource over `bytes` bytes starting at `base`, raw (unformatted)
// dword access: word 3 = 0x00020000 selects the 32-bit data format with no
// swizzle and no index stride.  Reads at or past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Buffer -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane
// i reads rsrc + voff + soff (voff per lane, soff wave-uniform) and writes
// lds_base + 16*i; lds_base must be wave-uniform (it goes to M0).
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds_base, int32_t voff,
                                                int32_t soff) {
  lds_poison_lane(lds_base);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}

// Waits for this wave's outstanding vector-memory loads (including direct
// global -> LDS copies).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Rotary embedding of 8 feature pairs: x1 holds bf16 features f .. f+7, x2
// the partners f+d/2 .. f+d/2+7; c0/c1 and s0/s1 the cos and sin of the 8
// angles.  (x1, x2) -> (x1 c - x2 s, x2 c + x1 s) in fp32, rounded to bf16.
__device__ __forceinline__ void rope8(u32x4& x1, u32x4& x2, f32x4 c0, f32x4 c1, f32x4 s0, f32x4 s1) {
  u32x4 y1, y2;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a0 = __builtin_bit_cast(float, x1[w] << 16), a1 = __builtin_bit_cast(float, x1[w] & 0xffff0000u);
    const float b0 = __builtin_bit_cast(float, x2[w] << 16), b1 = __builtin_bit_cast(float, x2[w] & 0xffff0000u);
    const float ca = w < 2 ? c0[2 * w] : c1[2 * w - 4], cb = w < 2 ? c0[2 * w + 1] : c1[2 * w - 3];
    const float sa = w < 2 ? s0[2 * w] : s1[2 * w - 4], sb = w < 2 ? s0[2 * w + 1] : s1[2 * w - 3];
    y1[w] = pack_bf16x2(fmaf(a0, ca, -b0 * sa), fmaf(a1, cb, -b1 * sb));
    y2[w] = pack_bf16x2(fmaf(b0, ca, a0 * sa), fmaf(b1, cb, a1 * sb));
  }
  x1 = y1;
  x2 = y2;
}

// Value of lane l^32 (the other half of the wave), via v_permlane32_swap:
// a VALU op, so no trip through the LDS crossbar.  swap(x, x) yields
// {x of lanes 0-31 in both halves, x of lanes 32-63 in both halves}.
__device__ __forceinline__ float max_across_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float min_across_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fminf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Lane-exchange helpers (wave64).
__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }
__device__ __forceinline__ float shfl(float x, int src) { return __shfl(x, src, 64); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Split-KV merge ("Optimizing Decoder Attention for LLMs on GPU", split-K
// decoding; the rescaling identity of "GPU learning day 24: Operator Fusion",
// section 3.4): with M = max_r lse_r (base 2),
//   O = sum_r 2^(lse_r - M) o_r / sum_r 2^(lse_r - M).
// Partial r's log-sum-exp is lse[r * ls]; this lane's PER output elements of
// it are po[r * ps + e * ES].
constexpr int kMergeBatch = 16;   // partials whose output loads are issued together
constexpr int kMergeWaves = 4;    // waves of a combine workgroup

// One wave over partials 0 .. nr-1: M, the weight sum W = sum_r 2^(lse_r - M)
// and acc = sum_r 2^(lse_r - M) o_r (M = -inf, W = 0, acc = 0 when nr == 0).
// The lanes read the log-sum-exps in parallel and reduce M and W across the
// wave; the outputs are accumulated kMergeBatch partials at a time with their
// loads issued together (the loads past nr are skipped and their weights are
// 0), so a merge of many partials is not a chain of dependent loads.
template <int PER, int ES>
__device__ __forceinline__ void merge_range(const float* lse, int64_t ls, const float* po, int64_t ps, int nr,
                                            float& M, float& W, float (&acc)[PER]) {
  const int lane = threadIdx.x & 63;
  // Outputs of partials c + j0 .. c + j0 + kMergeBatch - 1 (up to c + last).
  auto load_batch = [&](float (&v)[kMergeBatch][PER], int c, int j0, int last) {
#pragma unroll
    for (int t = 0; t < kMergeBatch; ++t) {
#pragma unroll
      for (int e = 0; e < PER; ++e) v[t][e] = 0.f;
      if (j0 + t > last) continue;   // uniform across the wave
      const float* src = po + (int64_t)(c + j0 + t) * ps;
      if constexpr (ES == 1 && PER == 4) {
        const float4 x = *reinterpret_cast<const float4*>(src);
        v[t][0] = x.x; v[t][1] = x.y; v[t][2] = x.z; v[t][3] = x.w;
      } else if constexpr (ES == 1 && PER == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        v[t][0] = x.x; v[t][1] = x.y;
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[t][e] = src[e * ES];
      }
    }
  };
  // The first 64 log-sum-exps and the first batch of outputs are loaded
  // together, before the maximum is known (the outputs do not depend on it),
  // so a merge of a few partials waits for one round of loads.  The batch's
  // loads past the last partial re-read it (their weights are 0), which keeps
  // them free of branches.
  const float l0 = lane < nr ? lse[(int64_t)lane * ls] : kNegInf;
  float v0[kMergeBatch][PER];
  if (nr > 0) {
    const int last0 = min(kMergeBatch, nr) - 1;
#pragma unroll
    for (int t = 0; t < kMergeBatch; ++t) {
      const float* src = po + (int64_t)min(t, last0) * ps;
      if constexpr (ES == 1 && PER == 4) {
        const float4 x = *reinterpret_cast<const float4*>(src);
        v0[t][0] = x.x; v0[t][1] = x.y; v0[t][2] = x.z; v0[t][3] = x.w;
      } else if constexpr (ES == 1 && PER == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        v0[t][0] = x.x; v0[t][1] = x.y;
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) v0[t][e] = src[e * ES];
      }
    }
  }
  M = l0;
  for (int r = lane + 64; r < nr; r += 64) M = fmaxf(M, lse[(int64_t)r * ls]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, shfl_xor(M, o));
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  W = 0.f;
  for (int c = 0; c < nr; c += 64) {
    const int r = c + lane;
    const float lr = c == 0 ? l0 : (r < nr ? lse[(int64_t)r * ls] : kNegInf);
    const float w = r < nr ? exp2_fast(lr - M) : 0.f;   // weight of partial c + lane
    W += w;
    const int last = min(64, nr - c) - 1;
    for (int j0 = 0; j0 <= last; j0 += kMergeBatch) {
      float v[kMergeBatch][PER];
      if (c == 0 && j0 == 0) {
#pragma unroll
        for (int t = 0; t < kMergeBatch; ++t)
#pragma unroll
          for (int e = 0; e < PER; ++e) v[t][e] = v0[t][e];
      } else {
        load_batch(v, c, j0, last);
      }
#pragma unroll
      for (int t = 0; t < kMergeBatch; ++t) {
        const float wt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j0 + t));
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(wt, v[t][e], acc[e]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) W += shfl_xor(W, o);
}

template <int PER, int NW>
struct MergeShared {
  float m[NW];
  float w[NW];
  float acc[NW][PER][64];
};

// A combine workgroup of NW waves (1 or kMergeWaves) merges nr partials:
// with one wave, or below 64 partials, wave 0 alone; otherwise each wave a
// contiguous share (at least 16 partials), the shares joined by the same
// identity through LDS.  nr must be the same for the whole workgroup.
// Returns the weight sum W relative to the overall maximum and leaves acc in
// wave 0's lanes (O = acc / W; W = 0 when nr == 0); the other waves' results
// are not meaningful.
template <int PER, int ES, int NW>
__device__ __forceinline__ float merge_partials(const float* lse, int64_t ls, const float* po, int64_t ps, int nr,
                                               float (&acc)[PER], MergeShared<PER, NW>& sh) {
  const int wave = NW == 1 ? 0 : threadIdx.x >> 6, lane = threadIdx.x & 63;
  float M, W;
  if (NW == 1 || nr < 64) {
    merge_range<PER, ES>(lse, ls, po, ps, wave == 0 ? nr : 0, M, W, acc);
    return W;
  }
  const int r0 = (int)((int64_t)nr * wave / NW);
  const int r1 = (int)((int64_t)nr * (wave + 1) / NW);
  merge_range<PER, ES>(lse + r0 * ls, ls, po + r0 * ps, ps, r1 - r0, M, W, acc);
  if (lane == 0) {
    sh.m[wave] = M;
    sh.w[wave] = W;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) sh.acc[wave][e][lane] = acc[e];
  __syncthreads();
  float Mt = sh.m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mt = fmaxf(Mt, sh.m[w]);
  float Wt = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float sc = exp2_fast(sh.m[w] - Mt);
    Wt = fmaf(sc, sh.w[w], Wt);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(sc, sh.acc[w][e][lane], acc[e]);
  }
  return Wt;
}

}  // namespace attn

// decode_f32.hip -- single-query attention over an fp32 KV cache.
//
// The same split-KV decode as decode_bf16.hip ("Optimizing Decoder Attention
// for LLMs on GPU": one query per head against every cached token, each K/V
// element read once; Flash-Decoding chunks merged with the rescaling identity
// of "GPU learning day 24: Operator Fusion", section 3.4), for inputs and
// output in fp32.  Every product and sum stays in fp32, so the result meets
// the fp32 bar (1e-5 relative) rather than the bf16 one.
//
// Kernels
//   decode_split_f32<D>    one workgroup per (split, query head, batch): a
//                          streaming dot product on the vector ALU (no
//                          contraction is dense enough here for the matrix
//                          cores; with query groups each query head streams
//                          its KV head's rows itself, so K/V is read once
//                          per query head, mostly from L2 for the later ones).
//   decode_combine_f32<D, NW>  merges a head's partials into O with one
//                          wave, or four that share 64 or more partials
//                          (skipped when every head has a single split).
//
// Partials share the bf16 decode's workspace layout of its chunked pass:
// part_o [B, Hq, n_split, d] normalised, part_lse [B, Hq, n_split] in base 2.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// First element of key row j of head (b, hk): the contiguous cache
// [B, Hkv, Skv, d] or the page that holds row j (table entries clamped to the
// pool).  A wave's rows of one iteration are consecutive rows of one page:
// iterations start at multiples of their key count (16 or 32) inside a chunk,
// chunks start at multiples of 256 keys, and page sizes are multiples of 128.
template <int D>
__device__ __forceinline__ const float* kv_row_f32(const void* t, const DecodeParams& p, int b, int hk, int j) {
  const float* base = static_cast<const float*>(t);
  if (!p.block_table) return base + (((int64_t)b * p.Hkv + hk) * p.Skv + j) * D;
  int pg = p.block_table[(int64_t)b * p.max_blocks + j / p.page_size];
  pg = min(max(pg, 0), p.num_pages - 1);
  return base + (((int64_t)pg * p.Hkv + hk) * p.page_size + j % p.page_size) * D;
}

// Lane layout: a key row is D/4 16-byte pieces (4 floats); LPK = D/4 lanes
// cover one key and a load instruction covers KPI = 64/LPK consecutive keys
// (1 KiB).  Per iteration a wave handles 8 instructions' worth of keys.  The
// 8 partial dot products of a lane are summed over the LPK lanes of its key
// group by a butterfly, which leaves each key's score in all of them.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_f32(DecodeParams p) {
  constexpr int LPK = D / 4;          // lanes per key row
  constexpr int KPI = 64 / LPK;       // keys per load instruction
  constexpr int KB = 8 * KPI;         // keys per wave iteration

  __shared__ float mrg_m[kWaves], mrg_l[kWaves];
  __shared__ float mrg_o[kWaves][D];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (p.Hq / p.Hkv);
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);
  const int c0 = split * p.chunk;
  float* orow = static_cast<float*>(p.o) + ((int64_t)b * p.Hq + h) * D;
  if (c0 >= n) {
    if (p.n_split == 1)   // no key: O = 0
      for (int d = threadIdx.x; d < D; d += kThreads) orow[d] = 0.f;
    return;
  }
  const int c1 = min(c0 + p.chunk, n);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane / LPK;          // key within an instruction's group
  const int dc = lane % LPK;          // 4-float feature chunk
  const f32x4 qv = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) +
                                                    ((int64_t)b * p.Hq + h) * D + 4 * dc);

  float m = kNegInf, lsum = 0.f;
  f32x4 o = {0.f, 0.f, 0.f, 0.f};

  for (int base = c0 + wave * KB; base < c1; base += kWaves * KB) {
    const float* kp = kv_row_f32<D>(p.k, p, b, hk, base);   // rows base .. base+KB-1
    const float* vp = kv_row_f32<D>(p.v, p, b, hk, base);
    f32x4 kr[8], vr[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = min(base + u * KPI + kg, c1 - 1) - base;
      kr[u] = *reinterpret_cast<const f32x4*>(kp + key * D + 4 * dc);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = min(base + u * KPI + kg, c1 - 1) - base;
      vr[u] = *reinterpret_cast<const f32x4*>(vp + key * D + 4 * dc);
    }
    float s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float a = qv[0] * kr[u][0];
      a = fmaf(qv[1], kr[u][1], a);
      a = fmaf(qv[2], kr[u][2], a);
      a = fmaf(qv[3], kr[u][3], a);
#pragma unroll
      for (int msk = 1; msk < LPK; msk <<= 1) a += shfl_xor(a, msk);
      const int key = base + u * KPI + kg;
      s[u] = key < c1 ? a * p.scale_log2 : kNegInf;
    }
    // wave max over the iteration's keys (the lanes of a group agree)
    float t = s[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) t = fmaxf(t, s[u]);
#pragma unroll
    for (int msk = LPK; msk < 64; msk <<= 1) t = fmaxf(t, shfl_xor(t, msk));
    const float m_new = fmaxf(m, t);            // finite: the iteration has a valid key
    const float alpha = exp2_fast(m - m_new);
    m = m_new;
    float psum = 0.f;
    o *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float pu = exp2_fast(s[u] - m_new);
      psum += pu;
      o[0] = fmaf(pu, vr[u][0], o[0]);
      o[1] = fmaf(pu, vr[u][1], o[1]);
      o[2] = fmaf(pu, vr[u][2], o[2]);
      o[3] = fmaf(pu, vr[u][3], o[3]);
    }
    lsum = lsum * alpha + psum;
  }

  // Sum over the key groups of the wave (each group's lanes share m, l).
#pragma unroll
  for (int msk = LPK; msk < 64; msk <<= 1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] += shfl_xor(o[e], msk);
    lsum += shfl_xor(lsum, msk);
  }
  if (lane == 0) {
    mrg_m[wave] = m;
    mrg_l[wave] = lsum;
  }
  if (lane < LPK) *reinterpret_cast<f32x4*>(&mrg_o[wave][4 * dc]) = o;
  __syncthreads();
  if (wave == 0) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg_m[w]);
    float L = 0.f, wgt[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wgt[w] = mrg_m[w] == kNegInf ? 0.f : exp2_fast(mrg_m[w] - M);
      L += wgt[w] * mrg_l[w];
    }
    const int64_t prow = ((int64_t)b * p.Hq + h) * p.n_split + split;
    for (int d = lane; d < D; d += 64) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) acc = fmaf(wgt[w], mrg_o[w][d], acc);
      if (p.n_split == 1) orow[d] = acc / L;
      else p.part_o[prow * D + d] = acc / L;
    }
    if (lane == 0 && p.n_split > 1) p.part_lse[prow] = M + log2_fast(L);
  }
}

// Merge of a head's partials: the splits that start below the length.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_combine_f32(DecodeParams p) {
  __shared__ MergeShared<D / 64, NW> sh;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);
  const int ns = (n + p.chunk - 1) / p.chunk;
  float* orow = static_cast<float*>(p.o) + ((int64_t)b * p.Hq + h) * D;
  const int64_t prow0 = ((int64_t)b * p.Hq + h) * p.n_split;
  float acc[D / 64];
  const float W = merge_partials<D / 64, 64, NW>(p.part_lse + prow0, 1, p.part_o + prow0 * D + lane, D, ns, acc, sh);
  if (threadIdx.x >= 64) return;   // wave 0 holds the result
#pragma unroll
  for (int e = 0; e < D / 64; ++e) orow[lane + 64 * e] = ns > 0 ? acc[e] / W : 0.f;
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_f32<D>), dim3(p.n_split, p.Hq, p.B), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  // four waves share a head's partials when there may be 64 or more
  if (p.n_split >= 64)
    hipLaunchKernelGGL((decode_combine_f32<D, kMergeWaves>), dim3(p.Hq, p.B), dim3(64 * kMergeWaves), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_combine_f32<D, 1>), dim3(p.Hq, p.B), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t stream) {
  if (p.d == 256) return launch_d<256>(p, stream);
  return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace attn

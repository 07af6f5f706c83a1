// decode_bf16.hip -- single-query attention over a bf16 KV cache.
//
// Decoding as described in "Optimizing Decoder Attention for LLMs on GPU"
// (magmadev.ru): one new query per head attends to every cached token, and
// the step is bound by reading the cache, so each K/V element is read from
// device memory exactly once per step.  The cache's sequence dimension is cut
// into chunks processed in parallel (Flash-Decoding, "GPU learning day 24:
// Operator Fusion", FAQ Q4); every chunk leaves a normalised partial output
// and its log-sum-exp, and a second kernel merges the partials with the
// rescaling identity of that page's section 3.4 loop.
//
// Kernels
//   decode_split_valu<D>     one query head per KV head (no reuse of K/V
//                            across queries: a streaming dot product, so the
//                            vector ALU is the right unit).
//   decode_split_balanced<D, G, EXACT>  G >= 2 query heads share each KV
//                            head, at most 2048 sequences: the queries form a
//                            small matrix and QK^T and PV run on
//                            v_mfma_f32_16x16x32_bf16 with the group padded to
//                            16 columns; a persistent pass over equal units of
//                            128 keys, with K and V staged per wave in LDS
//                            and each wave's next copies in flight while it
//                            computes (two workgroups per compute unit, one
//                            at d = 256).  decode_combine_balanced<D, G,
//                            EXACT, NW> merges.
//   decode_split_mfma<D, G, EXACT>  the same contraction on a grid of
//                            (chunk, KV head, batch) workgroups, for larger
//                            batches.
//   EXACT: groups of exactly G = 2, 4, 8 or 16 query heads.  Otherwise any
//   group size: each KV head's group is cut into column blocks of at most 16
//   query heads (virtual KV heads, see GroupMap), each reading the KV head
//   once, and G is the padded capacity (4, 8 or 16) of a block.
//   decode_combine<D, NW>    merges the partials of one (batch, query head)
//                            with NW = 1 or 4 waves (four share the partials
//                            of heads that may have more than 64); not
//                            launched when every head has a single split
//                            (decode_split_valu then writes O itself).
//
// Partial results are fp32; the log-sum-exp is kept in base-2 units
// (scores are scaled by scale * log2(e)).  Chunks that start at or beyond a
// sequence's length do no work and write nothing; the combine kernel derives
// the number of valid chunks from the same length.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Waits until at most N of this wave's vector-memory loads are outstanding
// (loads complete in issue order, so the earliest ones have landed).
template <int N>
__device__ __forceinline__ void wait_vmem_below() {
  static_assert(N >= 0 && N < 64, "vmcnt takes 0..63");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until this wave's LDS reads have returned their data.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LDS byte address of a generic pointer into shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// The score MFMA's K operand from LDS: 16-byte reads at a[ks] and a[ks] + HALF
// (the same slots 16 rows further on) into x0[ks] and x1[ks] for 4 k-steps,
// in one block that waits for its own reads.  The compiler then sees no LDS
// read here and inserts no wait for direct copies still in flight into other
// LDS buffers (it cannot tell those buffers apart and would wait for every
// copy); the caller waits for the copies into this buffer itself.
template <int HALF>
__device__ __forceinline__ void lds_read_k4(u32x4* x0, u32x4* x1, const uint32_t* a) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:%12\n\t"
      "ds_read_b128 %2, %9\n\t"
      "ds_read_b128 %3, %9 offset:%12\n\t"
      "ds_read_b128 %4, %10\n\t"
      "ds_read_b128 %5, %10 offset:%12\n\t"
      "ds_read_b128 %6, %11\n\t"
      "ds_read_b128 %7, %11 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x0[0]), "=&v"(x1[0]), "=&v"(x0[1]), "=&v"(x1[1]), "=&v"(x0[2]), "=&v"(x1[2]),
        "=&v"(x0[3]), "=&v"(x1[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "n"(HALF)
      : "memory");
}

template <int KS, int HALF>
__device__ __forceinline__ void lds_read_k(u32x4 (&x)[2][KS], const uint32_t (&a)[KS]) {
  static_assert(KS == 2 || KS == 4 || KS == 8, "d = 64, 128 or 256");
  if constexpr (KS >= 4) {
#pragma unroll
    for (int c = 0; c < KS; c += 4) lds_read_k4<HALF>(&x[0][c], &x[1][c], &a[c]);
  } else {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %5\n\t"
        "ds_read_b128 %3, %5 offset:%6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0][0]), "=&v"(x[1][0]), "=&v"(x[0][1]), "=&v"(x[1][1])
        : "v"(a[0]), "v"(a[1]), "n"(HALF)
        : "memory");
  }
}

// The PV MFMA's V^T operand from LDS: for output tile t, transposed 4-row
// reads at a[t] (rows 0..15 of the step) into lo[t] and at a[t] + HALF (rows
// 16..31) into hi[t], 8 tiles in one block that waits for its own reads (for
// the same reason as lds_read_k).
template <int HALF>
__device__ __forceinline__ void lds_read_vt8(u32x2* lo, u32x2* hi, const uint32_t* a) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:%24\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:%24\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:%24\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%24\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:%24\n\t"
      "ds_read_b64_tr_b16 %10, %21\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:%24\n\t"
      "ds_read_b64_tr_b16 %12, %22\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:%24\n\t"
      "ds_read_b64_tr_b16 %14, %23\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:%24\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
        "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5]),
        "=&v"(lo[6]), "=&v"(hi[6]), "=&v"(lo[7]), "=&v"(hi[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "n"(HALF)
      : "memory");
}

template <int DT, int HALF>
__device__ __forceinline__ void lds_read_vt(u32x2 (&lo)[DT], u32x2 (&hi)[DT], const uint32_t (&a)[DT]) {
  static_assert(DT == 4 || DT == 8 || DT == 16, "d = 64, 128 or 256");
  if constexpr (DT >= 8) {
#pragma unroll
    for (int c = 0; c < DT; c += 8) lds_read_vt8<HALF>(&lo[c], &hi[c], &a[c]);
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
          "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "n"(HALF)
        : "memory");
  }
}

// Read-only int32 from device memory through the constant address space: a
// wave-uniform address becomes a scalar load, which waits on no vector load.
__device__ __forceinline__ int32_t ld_const(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// First element of key row j of head (b, hk) in tensor t (K or V): the
// contiguous cache [B, Hkv, Skv, d], or the page that holds row j.  Every
// step of the split kernels covers at most 64 keys starting at a multiple of
// its size inside a kDecodeUnit-aligned block, and page sizes are multiples
// of kDecodeUnit, so a step's rows are consecutive rows of one page: the
// kernels look the page up once per step and address rows from there.
// Table entries are clamped to the pool, so no entry can address memory
// outside it.
template <int D>
__device__ __forceinline__ const uint16_t* kv_row(const void* t, const DecodeParams& p, int b, int hk,
                                                  int j) {
  const uint16_t* base = static_cast<const uint16_t*>(t);
  if (!p.block_table) return base + (((int64_t)b * p.Hkv + hk) * p.Skv + j) * D;
  int pg = ld_const(p.block_table + (int64_t)b * p.max_blocks + j / p.page_size);
  pg = min(max(pg, 0), p.num_pages - 1);
  return base + (((int64_t)pg * p.Hkv + hk) * p.page_size + j % p.page_size) * D;
}

// Cross-wave merge of (m, l, o[D]) held by each wave's lanes, then the
// partial is written by wave 0.  o_lane(d) gives this lane's share of o[d]
// for the dims it owns (already summed within the wave).
template <int D>
struct WaveMerge {
  float m[kWaves];
  float l[kWaves];
  float o[kWaves][D];
};

// ---------------------------------------------------------------------------
// G = 1: vector-ALU split kernel.
//
// Lane layout: a key row is D/8 16-byte pieces; LPK = D/8 lanes cover one key
// and a wave load instruction covers KPI = 64/LPK consecutive keys (1 KiB,
// fully coalesced).  Per iteration a wave handles 8 instructions' worth of
// keys (KB = 8*KPI).  The 8 partial dot products per lane are reduced across
// the LPK lanes of a key with a halving exchange, which leaves every key's
// full score in DUP = LPK/8 lanes.
//
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_valu(DecodeParams p) {
  constexpr int LPK = D / 8;          // lanes per key row
  constexpr int KPI = 64 / LPK;       // keys per load instruction
  constexpr int KB = 8 * KPI;         // keys per wave iteration
  constexpr int DUP = LPK / 8;        // lanes holding each reduced score (1, 2 or 4)

  __shared__ WaveMerge<D> merge;

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);
  const int c0 = split * p.chunk;
  // One split per head: this workgroup writes O itself (no combine pass).
  uint16_t* orow = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + h) * D;
  if (c0 >= n) {
    if (p.n_split == 1)   // no key: O = 0
      for (int d = threadIdx.x; d < D; d += kThreads) orow[d] = 0;
    return;
  }
  const int c1 = min(c0 + p.chunk, n);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane / LPK;          // key within an instruction's group
  const int dc = lane % LPK;          // 16-byte feature chunk
  const u32x4 qv = ld16(static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + h) * D + 8 * dc);

  // Which of the 8 keys of this lane's group its reduced score belongs to.
  const int my_u = (lane / DUP) & 7;

  float m = kNegInf, lsum = 0.f;
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  for (int base = c0 + wave * KB; base < c1; base += kWaves * KB) {
    const uint16_t* kp = kv_row<D>(p.k, p, b, h, base);   // rows base .. base+KB-1
    const uint16_t* vp = kv_row<D>(p.v, p, b, h, base);
    u32x4 kr[8], vr[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = min(base + u * KPI + kg, c1 - 1) - base;
      kr[u] = ld16_stream(kp + key * D + 8 * dc);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = min(base + u * KPI + kg, c1 - 1) - base;
      vr[u] = ld16_stream(vp + key * D + 8 * dc);
    }
    // partial dots over this lane's 8 features
    float part[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[w]), as_bf16x2(kr[u][w]), a, false);
      part[u] = a;
    }
    // halving exchange: 8 values over LPK lanes -> one full score per lane
    // (pair).  Masks LPK/2, LPK/4, LPK/8 each halve the values a lane keeps;
    // with LPK = 16 a last exchange over mask 1 completes the sum.
    {
      constexpr int MA = LPK / 2, MB = LPK / 4, MC = LPK / 8;
      const bool ba = lane & MA;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float send = ba ? part[t] : part[t + 4];
        const float keep = ba ? part[t + 4] : part[t];
        part[t] = keep + shfl_xor(send, MA);
      }
      const bool bb = lane & MB;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float send = bb ? part[t] : part[t + 2];
        const float keep = bb ? part[t + 2] : part[t];
        part[t] = keep + shfl_xor(send, MB);
      }
      const bool bc = lane & MC;
      const float send = bc ? part[0] : part[1];
      const float keep = bc ? part[1] : part[0];
      part[0] = keep + shfl_xor(send, MC);
#pragma unroll
      for (int msk = LPK / 16; msk >= 1; msk >>= 1) part[0] += shfl_xor(part[0], msk);
    }
    float s = part[0];
    const int my_key = base + my_u * KPI + kg;
    s = (my_key < c1) ? s * p.scale_log2 : kNegInf;

    // wave max
    float t = s;
#pragma unroll
    for (int msk = 1; msk < 64; msk <<= 1) t = fmaxf(t, shfl_xor(t, msk));
    const float m_new = fmaxf(m, t);
    const float alpha = exp2_fast(m - m_new);   // m_new is finite: the block has a valid key
    const float pr = exp2_fast(s - m_new);
    m = m_new;
    lsum = lsum * alpha + pr;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
    // o += sum_u p_u v_u over this lane's 8 keys
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int src = kg * LPK + u * DUP;
      const float pu = shfl(pr, src);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        o[2 * w] = fmaf(pu, bf16_lo(vr[u][w]), o[2 * w]);
        o[2 * w + 1] = fmaf(pu, bf16_hi(vr[u][w]), o[2 * w + 1]);
      }
    }
  }

  // Reduce within the wave: o over the KPI key groups, l over all lanes.
#pragma unroll
  for (int msk = LPK; msk < 64; msk <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += shfl_xor(o[e], msk);
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) lsum += shfl_xor(lsum, msk);
  lsum *= 1.0f / DUP;

  if (lane == 0) {
    merge.m[wave] = m;
    merge.l[wave] = lsum;
  }
  if (lane < LPK) {
#pragma unroll
    for (int e = 0; e < 8; ++e) merge.o[wave][8 * dc + e] = o[e];
  }
  __syncthreads();
  if (wave == 0) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, merge.m[w]);
    float L = 0.f, wgt[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      wgt[w] = merge.m[w] == kNegInf ? 0.f : exp2_fast(merge.m[w] - M);
      L += wgt[w] * merge.l[w];
    }
    const float invL = 1.f / L;
    const int64_t prow = ((int64_t)b * p.Hq + h) * p.n_split + split;
    for (int d = lane; d < D; d += 64) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) acc += wgt[w] * merge.o[w][d];
      if (p.n_split == 1) orow[d] = f32_to_bf16_bits(acc * invL);
      else p.part_o[prow * D + d] = acc * invL;
    }
    if (lane == 0 && p.n_split > 1) p.part_lse[prow] = M + log2_fast(L);
  }
}

// Query columns of virtual KV head vh: the KV head it reads, its first
// query head within the batch, and how many query heads it holds.  EXACT:
// groups of exactly G, one block per KV head.
template <int G, bool EXACT>
struct GroupMap {
  int hk, q0, g;
  __device__ __forceinline__ GroupMap(const DecodeParams& p, int vh) {
    if constexpr (EXACT) {
      hk = vh;
      q0 = vh * G;
      g = G;
    } else {
      hk = vh / p.kv_div;
      const int blk = vh - hk * p.kv_div;
      const int grp = p.Hq / p.Hkv;
      q0 = hk * grp + blk * p.cb;
      g = min(p.cb, grp - blk * p.cb);
    }
  }
};

// ---------------------------------------------------------------------------
// G >= 2: matrix-core split kernel.
//
// Per 32-key step a wave computes S^T (32 keys x 16 query rows, rows >= G are
// zero padding) with v_mfma_f32_16x16x32_bf16: K rows come straight from
// device memory as the A operand (lane = key row, 8 features), Q^T is a
// register-resident B operand.  Each lane then holds 8 keys of one query
// column, which is already the B-operand layout of O^T += V^T P^T under a
// fixed permutation of the 32 keys.  The wave stages its V rows in its own
// LDS region (coalesced 16-byte stores, rows swizzled by lds_swizzle) and
// reads V^T with the LDS transpose read, so no workgroup barrier is needed
// inside the loop.
// ---------------------------------------------------------------------------
// At d = 256 the fragments (K 64, V 64, O 64, Q 32 registers) and the rest
// exceed 256 registers, so one wave per SIMD (a 64.5 KiB workgroup per CU,
// 128 KiB of K and V in flight); d = 64 and 128 fit three.
template <int D, int G, bool EXACT>
__global__ __launch_bounds__(kThreads, (D == 256 ? 1 : 3)) void decode_split_mfma(DecodeParams p) {
  constexpr int KS = D / 32;          // k-steps of the score MFMA (32 features each)
  constexpr int DT = D / 16;          // 16-feature output tiles
  constexpr int SLOTS = D / 8;        // 16-byte slots per V row
  constexpr int VBYTES = 32 * D * 2;  // one wave's V block
  constexpr int VP = 32 * SLOTS / 64; // V pieces per lane per step

  // V staging during the loop; reused afterwards for the cross-wave merge.
  static_assert(kWaves * G * D * 4 <= kWaves * VBYTES, "merge buffer must fit the V buffers");
  __shared__ __attribute__((aligned(16))) unsigned char vbuf[kWaves][VBYTES];
  __shared__ float mrg_m[kWaves][16];
  __shared__ float mrg_l[kWaves][16];
  float (*mrg_o)[G][D] = reinterpret_cast<float (*)[G][D]>(&vbuf[0][0]);

  const int split = blockIdx.x, b = blockIdx.z;
  const GroupMap<G, EXACT> gm(p, blockIdx.y);
  const int hk = gm.hk;
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);
  const int c0 = split * p.chunk;
  if (c0 >= n) return;
  const int c1 = min(c0 + p.chunk, n);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qcol = lane & 15;          // query column (valid if < gm.g)
  const int grp = lane >> 4;           // 16-lane group

  // Q^T as B operand: lane (qcol, grp) holds Q[q0 + qcol][32*ks + 8*grp .. +7].
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + gm.q0) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (qcol < gm.g) w = ld16(qp + (int64_t)qcol * D + 32 * ks + 8 * grp);
      qreg[ks] = as_bf16x8(w);
    }
  }

  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{};
  float m = kNegInf, lsum = 0.f;
  unsigned char* vb = vbuf[wave];
  const uint32_t k_off = (uint32_t)(qcol * D * 2 + grp * 16);   // byte offset of this lane's K piece

  for (int base = c0 + wave * 32; base < c1; base += kWaves * 32) {
    // K as A operand: lane (row = lane%16, grp) -> K[base + 16*hlf + row][32*ks + 8*grp ..]
    // V rows of this step: coalesced pieces, row = piece / SLOTS.
    // A full step reads from a uniform base plus lane-constant offsets; the
    // last, partial step clamps rows to the chunk's last valid key.
    const uint16_t* kp = kv_row<D>(p.k, p, b, hk, base);   // rows base .. base+31
    const uint16_t* vp = kv_row<D>(p.v, p, b, hk, base);
    u32x4 kr[2][KS];
    u32x4 vr[VP];
    if (base + 32 <= c1) {
      const char* kb = reinterpret_cast<const char*>(kp);
      const char* vbs = reinterpret_cast<const char*>(vp);
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kr[hlf][ks] = ld16_stream(kb + k_off + hlf * 16 * D * 2 + ks * 64);
#pragma unroll
      for (int u = 0; u < VP; ++u) vr[u] = ld16_stream(vbs + lane * 16 + u * 1024);
    } else {
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int key = min(base + 16 * hlf + qcol, c1 - 1) - base;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kr[hlf][ks] = ld16_stream(kp + key * D + 32 * ks + 8 * grp);
      }
#pragma unroll
      for (int u = 0; u < VP; ++u) {
        const int piece = u * 64 + lane;
        const int row = piece / SLOTS, slot = piece % SLOTS;
        const int key = min(base + row, c1 - 1) - base;
        vr[u] = ld16_stream(vp + key * D + slot * 8);
      }
    }
    // S^T for keys [base, base+16) and [base+16, base+32)
    f32x4 sacc[2];
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf) {
      sacc[hlf] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        sacc[hlf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[hlf][ks]), qreg[ks], sacc[hlf], 0, 0, 0);
    }
    // stage V (wave-private LDS region, swizzled)
#pragma unroll
    for (int u = 0; u < VP; ++u) {
      const int piece = u * 64 + lane;
      const int row = piece / SLOTS, slot = piece % SLOTS;
      *reinterpret_cast<u32x4*>(vb + (row * SLOTS + (slot ^ (lds_swizzle(row) & (SLOTS - 1)))) * 16) = vr[u];
    }
    // lane holds keys base + 16*hlf + 4*grp + i for query qcol
    float tmax = kNegInf;
#pragma unroll
    for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = base + 16 * hlf + 4 * grp + i;
        const float s = key < c1 ? sacc[hlf][i] * p.scale_log2 : kNegInf;
        sacc[hlf][i] = s;
        tmax = fmaxf(tmax, s);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float m_new = fmaxf(m, tmax);            // finite: the step has a valid key
    const float alpha = exp2_fast(m - m_new);
    m = m_new;
    uint32_t w[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int hlf = e / 2, i0 = 2 * (e % 2);
      w[e] = pack_bf16x2(exp2_fast(sacc[hlf][i0] - m_new), exp2_fast(sacc[hlf][i0 + 1] - m_new));
      psum += bf16_lo(w[e]) + bf16_hi(w[e]);
    }
    lsum = lsum * alpha + psum;
    const bf16x8 pb = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] *= alpha;

    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T: the B operand's 8 keys are (4*grp + 0..3, 16 + 4*grp + 0..3)
    const int src = lane & 15;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int cidx = 16 * t + 4 * (src & 3);
      const int cslot = cidx >> 3, cbyte = (cidx & 7) * 2;
      const int r0 = 4 * grp + (src >> 2);
      const int r1 = r0 + 16;
      const u32x2 lo = lds_read_tr16x4(vb + (r0 * SLOTS + (cslot ^ (lds_swizzle(r0) & (SLOTS - 1)))) * 16 + cbyte);
      const u32x2 hi = lds_read_tr16x4(vb + (r1 * SLOTS + (cslot ^ (lds_swizzle(r1) & (SLOTS - 1)))) * 16 + cbyte);
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]}), pb, oacc[t], 0, 0, 0);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // l per query: sum over the 4 lane groups holding the same query column.
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  // O^T accumulator: lane (qcol, grp) holds features 16*t + 4*grp + i.
  if (lane < 16) {
    mrg_m[wave][qcol] = m;
    mrg_l[wave][qcol] = lsum;
  }
  __syncthreads();   // every wave is done with its V buffer before it is reused
  if (qcol < gm.g) {
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mrg_o[wave][qcol][16 * t + 4 * grp + i] = oacc[t][i];
  }
  __syncthreads();
  // merge the waves: thread tid handles (query, feature) pairs
  for (int idx = tid; idx < gm.g * D; idx += kThreads) {
    const int qi = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg_m[w][qi]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = mrg_m[w][qi] == kNegInf ? 0.f : exp2_fast(mrg_m[w][qi] - M);
      L += wt * mrg_l[w][qi];
      acc += wt * mrg_o[w][qi][d];
    }
    const int64_t prow = ((int64_t)b * p.Hq + gm.q0 + qi) * p.n_split + split;
    p.part_o[prow * D + d] = acc / L;
    if (d == 0) p.part_lse[prow] = M + log2_fast(L);
  }
}

// ---------------------------------------------------------------------------
// G >= 2, balanced: a persistent split pass over equal-size work units.
//
// With ragged lengths a grid of (split, head, batch) workgroups leaves many
// compute units idle at the end (short and empty splits).  Here the cache is
// cut into units of kDecodeUnit keys, ordered (batch, KV head, unit); unit
// counts per batch come from the lengths on the device, and every workgroup
// recomputes their prefix sum in LDS.  Workgroup w takes units
// [w*R, (w+1)*R), R = ceil(U / gridDim.x), walking across heads: runs of units
// of one head are merged on the fly, and each run ("segment") leaves one
// partial (o, base-2 lse) per query head, at the slot run_slot() gives it
// (fewer than B * H_kv + gridDim.x slots in all, whatever the lengths).  The
// combine kernel finds a head's segments from the same prefix sums and R.
// ---------------------------------------------------------------------------

// Partial slot of the run that starts at unit u of flattened head h = b *
// H_kv + g, with R units per workgroup.  A run starts at its head's first unit
// or at a multiple of R, so runs of one head have distinct u / R, and a later
// head's runs start at units no smaller than an earlier head's: h + u / R is
// distinct for every run and below B * H_kv + (number of workgroups).
__device__ __forceinline__ int run_slot(int h, int u, int R) { return h + u / R; }

// Exclusive prefix over batches of hv * ceil(n_b / kDecodeUnit) into pre[0..B]
// (pre[B] = total units; hv: the virtual KV heads).  All threads of the
// workgroup take part.
__device__ __forceinline__ void unit_prefix(const DecodeParams& p, int hv, int* pre, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = (p.B + kThreads - 1) / kThreads;      // batches per thread (<= 8)
  const int b0 = tid * per;
  int vals[kDecodeMaxBatch / kThreads];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kDecodeMaxBatch / kThreads; ++i) {
    int u = 0;
    if (i < per && b0 + i < p.B) {
      int n = p.Skv;
      if (p.kv_lens) n = min(max(p.kv_lens[b0 + i], 0), p.Skv);
      u = hv * ((n + kDecodeUnit - 1) / kDecodeUnit);
    }
    vals[i] = u;
    sum += u;
  }
  // inclusive scan of the per-thread sums within the wave
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  int run = base + incl - sum;                         // exclusive prefix of this thread
#pragma unroll
  for (int i = 0; i < kDecodeMaxBatch / kThreads; ++i) {
    if (i < per && b0 + i < p.B) pre[b0 + i] = run;
    run += vals[i];
  }
  if (tid == kThreads - 1) pre[p.B] = base + incl;
  __syncthreads();
}

template <int D, int G, bool EXACT>
__global__ __launch_bounds__(kThreads, decode_wg_per_cu(D)) void decode_split_balanced(DecodeParams p) {
  constexpr int KS = D / 32;          // k-steps of the score MFMA (32 features each)
  constexpr int DT = D / 16;          // 16-feature output tiles
  constexpr int SLOTS = D / 8;        // 16-byte slots per V row
  constexpr int VBYTES = 32 * D * 2;  // one wave's V block
  constexpr int VP = 32 * SLOTS / 64; // V pieces per lane per step

  static_assert(kWaves * G * D * 4 <= kWaves * VBYTES, "merge buffer must fit the V buffers");
  __shared__ __attribute__((aligned(16))) unsigned char vbuf[kWaves][VBYTES];
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[kWaves][VBYTES];
  __shared__ float mrg_m[kWaves][16];
  __shared__ float mrg_l[kWaves][16];
  __shared__ int wave_tot[kWaves];
  extern __shared__ int pre[];         // [B + 1], dynamic
  float (*mrg_o)[G][D] = reinterpret_cast<float (*)[G][D]>(&vbuf[0][0]);

  const int HV = EXACT ? p.Hkv : p.Hv;     // (virtual) KV heads: the units' head dimension
  const int CB = EXACT ? G : p.cb;        // partial slots per run
  unit_prefix(p, HV, pre, wave_tot);
  // Work coordinates are kept wave-uniform (scalar registers), so length and
  // page-table reads are scalar loads that never wait on the copies in flight.
  const int U = __builtin_amdgcn_readfirstlane(pre[p.B]);
  const int R = (U + (int)gridDim.x - 1) / (int)gridDim.x;
  int u = (int)blockIdx.x * R;
  const int uend = min(u + R, U);
  if (u >= uend) return;                               // uniform across the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qcol = lane & 15;          // query column (valid if < G)
  const int grp = lane >> 4;           // 16-lane group
  unsigned char* vb = vbuf[wave];
  unsigned char* kb = kbuf[wave];
  // LDS addresses of this lane's K-operand slots (row qcol, features
  // 32*ks + 8*grp .. +7).
  uint32_t k_addr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_addr[ks] = lds_addr(kb + (qcol * SLOTS + ((4 * ks + grp) ^ (lds_swizzle(qcol) & (SLOTS - 1)))) * 16);
  // LDS addresses of this lane's transposed V reads: output tile t, source
  // lane (lane & 15) names row 4*grp + (lane&15)/4 and columns 16*t +
  // 4*(lane%4) .. +3 (rows r and r + 16 share a swizzle).
  uint32_t v_addr[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const int src = lane & 15;
    const int cidx = 16 * t + 4 * (src & 3);
    const int cslot = cidx >> 3, cbyte = (cidx & 7) * 2;
    const int r0 = 4 * grp + (src >> 2);
    v_addr[t] = lds_addr(vb + (r0 * SLOTS + (cslot ^ (lds_swizzle(r0) & (SLOTS - 1)))) * 16 + cbyte);
  }
  // V copy w puts this lane's 16 bytes at LDS row v_row0 + w*kRowsPerCopy,
  // physical slot v_phys; the swizzle of that row picks the logical slot.
  constexpr int kRowsPerCopy = 1024 / (2 * D);
  const int v_row0 = (lane * 16) / (2 * D);
  const int v_phys = ((lane * 16) % (2 * D)) / 16;
  auto v_slot = [&](int w) {
    return v_phys ^ (lds_swizzle(v_row0 + w * kRowsPerCopy) & (SLOTS - 1));
  };

  // Locate unit u: batch b = last with pre[b] <= u (batches without units
  // have pre[b] == pre[b+1] and are skipped by taking the last such b).
  int lo = 0, hi = p.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (__builtin_amdgcn_readfirstlane(pre[mid]) <= u) lo = mid; else hi = mid - 1;
  }
  int b = lo;
  int pre_b = __builtin_amdgcn_readfirstlane(pre[b]);
  int units_b = (__builtin_amdgcn_readfirstlane(pre[b + 1]) - pre_b) / HV;
  int hk = (u - pre_b) / units_b;         // virtual KV head
  int k = (u - pre_b) % units_b;

  while (u < uend) {
    const GroupMap<G, EXACT> gm(p, hk);
    int n = p.Skv;
    if (p.kv_lens) n = min(max(ld_const(p.kv_lens + b), 0), p.Skv);
    const int seg_start = u;
    const int seg_end = min(uend, pre_b + (hk + 1) * units_b);

    // Q^T as B operand: lane (qcol, grp) holds Q[h0 + qcol][32*ks + 8*grp .. +7].
    bf16x8 qreg[KS];
    {
      const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + gm.q0) * D;
      u32x4 w[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        w[ks] = u32x4{0u, 0u, 0u, 0u};
        if (qcol < gm.g) w[ks] = ld16(qp + (int64_t)qcol * D + 32 * ks + 8 * grp);
      }
      // Use the values here, so the wait for the Q loads is placed now and
      // not before every score MFMA of the step loop.
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        asm volatile("" ::"v"(w[ks]));
        qreg[ks] = as_bf16x8(w[ks]);
      }
    }
    f32x4 oacc[DT];
#pragma unroll
    for (int t = 0; t < DT; ++t) oacc[t] = f32x4{};
    float m = kNegInf, lsum = 0.f;

    // This wave's steps in the segment: units k0 .. k0 + nst - 1, those whose
    // 32-key slice starts below the length.
    const int k0 = k;
    const int lim = n - wave * 32;
    const int nst = lim > 0 ? max(0, min(seg_end - seg_start, (lim + kDecodeUnit - 1) / kDecodeUnit - k0)) : 0;
    // K or V rows base .. base+31 straight into this wave's LDS region dst by
    // direct copies (copy w lands lane i at byte w*1024 + 16*i): each copy
    // reads whole rows, 1 KiB contiguous, where loading K into the MFMA
    // operand layout would touch 16 rows per instruction.  Rows past the
    // length repeat row n-1.
    auto issue = [&](unsigned char* dst, const void* t, int base) __attribute__((always_inline)) {
      const char* src = reinterpret_cast<const char*>(kv_row<D>(t, p, b, gm.hk, base));
      if (base + 32 <= n) {
#pragma unroll
        for (int w = 0; w < VP; ++w)
          global_to_lds16_stream(src + (v_row0 + w * kRowsPerCopy) * 2 * D + v_slot(w) * 16, dst + w * 1024);
      } else {
#pragma unroll
        for (int w = 0; w < VP; ++w) {
          const int key = min(base + v_row0 + w * kRowsPerCopy, n - 1) - base;
          global_to_lds16_stream(src + key * 2 * D + v_slot(w) * 16, dst + w * 1024);
        }
      }
    };
    // Software pipeline: a buffer is refilled with the next step's rows as
    // soon as this step has read it, so the next K copies fly during this
    // step's softmax and PV, and the next V copies during the next scores.
    // Outstanding copies are always K(i) then V(i), or V(i) then K(i+1).
    if (nst > 0) {
      issue(kb, p.k, k0 * kDecodeUnit + wave * 32);
      issue(vb, p.v, k0 * kDecodeUnit + wave * 32);
    }
    for (int i = 0; i < nst; ++i) {
      const int base = (k0 + i) * kDecodeUnit + wave * 32;
      const bool more = i + 1 < nst;
      wait_vmem_below<VP>();   // K(i) has landed (V(i) may be in flight)
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // K rows into the A-operand layout: lane (qcol, grp) takes row
      // 16*hlf + qcol, features 32*ks + 8*grp .. +7.
      // (Rows r and r + 16 share a swizzle, so the second half is 16 rows on.)
      u32x4 kr[2][KS];
      lds_read_k<KS, 16 * SLOTS * 16>(kr, k_addr);
      if (more) issue(kb, p.k, base + kDecodeUnit);   // the K reads have returned: refill
      f32x4 sacc[2];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        sacc[hlf] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sacc[hlf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[hlf][ks]), qreg[ks], sacc[hlf], 0, 0, 0);
      }
      // lane holds keys base + 16*hlf + 4*grp + i for query qcol
      float tmax = kNegInf;
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = base + 16 * hlf + 4 * grp + e;
          const float s = key < n ? sacc[hlf][e] * p.scale_log2 : kNegInf;
          sacc[hlf][e] = s;
          tmax = fmaxf(tmax, s);
        }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float m_new = fmaxf(m, tmax);            // finite: the slice has a valid key
      const float alpha = exp2_fast(m - m_new);
      m = m_new;
      uint32_t pw[4];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int hlf = e / 2, i0 = 2 * (e % 2);
        pw[e] = pack_bf16x2(exp2_fast(sacc[hlf][i0] - m_new), exp2_fast(sacc[hlf][i0 + 1] - m_new));
        psum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(pw[e]), kOnesBf16x2, psum, false);
      }
      lsum = lsum * alpha + psum;
      const bf16x8 pb = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;

      if (more) wait_vmem_below<VP>();   // V(i) has landed (K(i+1) may be in flight)
      else wait_vmem();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      u32x2 vlo[DT], vhi[DT];
      lds_read_vt<DT, 16 * SLOTS * 16>(vlo, vhi, v_addr);
#pragma unroll
      for (int t = 0; t < DT; ++t)
        oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{vlo[t][0], vlo[t][1], vhi[t][0], vhi[t][1]}),
                                                          pb, oacc[t], 0, 0, 0);
      if (more) {
        wait_lds();            // the V reads are in registers: refill the buffer
        issue(vb, p.v, base + kDecodeUnit);
      }
    }
    k = k0 + (seg_end - seg_start);
    u = seg_end;

    // Flush the segment: merge the waves, write one partial per query head.
    lsum += shfl_xor(lsum, 16);
    lsum += shfl_xor(lsum, 32);
    if (lane < 16) {
      mrg_m[wave][qcol] = m;
      mrg_l[wave][qcol] = lsum;
    }
    __syncthreads();   // every wave is done with its V buffer before it is reused
    if (qcol < gm.g) {
#pragma unroll
      for (int t = 0; t < DT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mrg_o[wave][qcol][16 * t + 4 * grp + i] = oacc[t][i];
    }
    __syncthreads();
    for (int idx = tid; idx < gm.g * D; idx += kThreads) {
      const int qi = idx / D, d = idx % D;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mrg_m[w][qi]);
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wt = mrg_m[w][qi] == kNegInf ? 0.f : exp2_fast(mrg_m[w][qi] - M);
        L += wt * mrg_l[w][qi];
        acc += wt * mrg_o[w][qi][d];
      }
      const int64_t slot = (int64_t)run_slot(b * HV + hk, seg_start, R) * CB + qi;
      p.part_o[slot * D + d] = acc / L;
      if (d == 0) p.part_lse[slot] = M + log2_fast(L);
    }
    __syncthreads();   // the merge buffer (aliasing the V buffers) is free again

    // next head: skip batches without units
    k = 0;
    if (++hk == HV) {
      hk = 0;
      do { ++b; } while (b < p.B && __builtin_amdgcn_readfirstlane(pre[b + 1]) == __builtin_amdgcn_readfirstlane(pre[b]));
      if (b < p.B) {
        pre_b = __builtin_amdgcn_readfirstlane(pre[b]);
        units_b = (__builtin_amdgcn_readfirstlane(pre[b + 1]) - pre_b) / HV;
      }
    }
  }
}

// Combine for the balanced pass: (virtual) head (b, g) owns units [hs, he);
// its segments start at hs and at every multiple of R inside (hs, he).
template <int D, int G, bool EXACT, int NW>
__global__ __launch_bounds__(64 * NW) void decode_combine_balanced(DecodeParams p) {
  __shared__ MergeShared<D / 64, NW> sh;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int HV = EXACT ? p.Hkv : p.Hv;
  const int CB = EXACT ? G : p.cb;
  int g, qi;                            // virtual KV head, column within its block
  if constexpr (EXACT) {
    g = hq / G;
    qi = hq % G;
  } else {
    const int grp = p.Hq / p.Hkv, hkr = hq / grp, j = hq - hkr * grp;
    g = hkr * p.kv_div + j / p.cb;
    qi = j % p.cb;
  }
  // units before batch b, and in total (lane-strided sums over batches)
  int before = 0, total = 0, units_b = 0;
  for (int bb = lane; bb < p.B; bb += 64) {
    int n = p.Skv;
    if (p.kv_lens) n = min(max(p.kv_lens[bb], 0), p.Skv);
    const int ub = (n + kDecodeUnit - 1) / kDecodeUnit;
    total += ub;
    if (bb < b) before += ub;
    if (bb == b) units_b = ub;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    before += __shfl_xor(before, o, 64);
    total += __shfl_xor(total, o, 64);
    units_b += __shfl_xor(units_b, o, 64);
  }
  const int U = total * HV;
  const int R = (U + p.n_wg - 1) / p.n_wg;
  const int hs = before * HV + g * units_b, he = hs + units_b;
  uint16_t* orow = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + hq) * D;
  constexpr int PER = D / 64;
  // The head's runs start at hs and at every multiple of R inside (hs, he),
  // so their slots run_slot(head, s, R) are consecutive: head + hs/R ..
  // head + (he-1)/R.
  const int nr = he > hs ? (he - 1) / R - hs / R + 1 : 0;
  const int64_t slot0 = (int64_t)run_slot(b * HV + g, hs, R) * CB + qi;
  float acc[PER];
  const float Wsum = merge_partials<PER, 1, NW>(p.part_lse + slot0, CB, p.part_o + slot0 * D + PER * lane,
                                                (int64_t)CB * D, nr, acc, sh);
  if (threadIdx.x >= 64) return;   // wave 0 holds the result
  const float inv = nr > 0 ? 1.f / Wsum : 0.f;
  if constexpr (PER == 4) {
    *reinterpret_cast<u32x2*>(orow + 4 * lane) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                                       pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  } else if constexpr (PER == 2) {
    reinterpret_cast<uint32_t*>(orow)[lane] = pack_bf16x2(acc[0] * inv, acc[PER - 1] * inv);
  } else {
    orow[lane] = f32_to_bf16_bits(acc[0] * inv);
  }
}

// ---------------------------------------------------------------------------
// Combine: O = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max_s lse_s.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void decode_combine(DecodeParams p) {
  __shared__ MergeShared<D / 64, NW> sh;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);
  const int ns = (n + p.chunk - 1) / p.chunk;
  uint16_t* orow = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + h) * D;
  const int64_t prow0 = ((int64_t)b * p.Hq + h) * p.n_split;
  constexpr int PER = D / 64;
  float acc[PER];
  const float W = merge_partials<PER, 1, NW>(p.part_lse + prow0, 1, p.part_o + prow0 * D + PER * lane, D, ns, acc, sh);
  if (threadIdx.x >= 64) return;   // wave 0 holds the result
  const float inv = ns > 0 ? 1.f / W : 0.f;
  if constexpr (PER == 4) {
    *reinterpret_cast<u32x2*>(orow + 4 * lane) = u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                                       pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  } else if constexpr (PER == 2) {
    reinterpret_cast<uint32_t*>(orow)[lane] = pack_bf16x2(acc[0] * inv, acc[PER - 1] * inv);
  } else {
    orow[lane] = f32_to_bf16_bits(acc[0] * inv);
  }
}

// Combine workgroups: kMergeWaves waves when a head may have more than 64
// partials (the waves share them), else one.  The chunked passes know their
// split count.  The balanced pass's runs per head are at most its units per
// head, ceil(S_kv / kDecodeUnit), and are few whenever many heads share the
// grid, so it takes four waves only for long caches over at most 1024 query
// heads (four waves per head cost a few µs over 4096 heads).
template <int D>
hipError_t launch_combine(const DecodeParams& p, hipStream_t stream) {
  if (p.n_split >= 64)
    hipLaunchKernelGGL((decode_combine<D, kMergeWaves>), dim3(p.Hq, p.B), dim3(64 * kMergeWaves), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_combine<D, 1>), dim3(p.Hq, p.B), dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G, bool EXACT>
hipError_t launch_balanced(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_balanced<D, G, EXACT>), dim3(p.n_wg), dim3(kThreads), (p.B + 1) * sizeof(int),
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool wide = (p.Skv + kDecodeUnit - 1) / kDecodeUnit > 64 && (int64_t)p.B * p.Hq <= 1024;
  if (wide)
    hipLaunchKernelGGL((decode_combine_balanced<D, G, EXACT, kMergeWaves>), dim3(p.Hq, p.B), dim3(64 * kMergeWaves),
                       0, stream, p);
  else
    hipLaunchKernelGGL((decode_combine_balanced<D, G, EXACT, 1>), dim3(p.Hq, p.B), dim3(64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int G, bool EXACT>
hipError_t launch_group(const DecodeParams& p, hipStream_t stream) {
  if (p.n_wg > 0) return launch_balanced<D, G, EXACT>(p, stream);
  hipLaunchKernelGGL((decode_split_mfma<D, G, EXACT>), dim3(p.n_split, p.Hv, p.B), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_combine<D>(p, stream);
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  if (G == 1) {
    hipLaunchKernelGGL((decode_split_valu<D>), dim3(p.n_split, p.Hq, p.B), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;   // one split: the split pass wrote O
    return launch_combine<D>(p, stream);
  }
  {
  if (p.kv_div == 1 && p.cb == G) {
    switch (G) {
      case 2: return launch_group<D, 2, true>(p, stream);
      case 4: return launch_group<D, 4, true>(p, stream);
      case 8: return launch_group<D, 8, true>(p, stream);
      case 16: return launch_group<D, 16, true>(p, stream);
      default: break;
    }
  }
  // any other group: column blocks of cb <= 16 query heads, padded to 4, 8 or 16
  if (p.cb <= 4) return launch_group<D, 4, false>(p, stream);
  if (p.cb <= 8) return launch_group<D, 8, false>(p, stream);
  if (p.cb <= 16) return launch_group<D, 16, false>(p, stream);
  return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
  if (p.d == 256) return launch_d<256>(p, stream);
  return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace attn


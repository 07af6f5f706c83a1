// prefill_d256.hip -- bf16 attention forward at head dimension 256 on gfx950.
//
// The same tiled online-softmax loop as prefill_bf16.hip ("GPU learning day
// 24: Operator Fusion", section 3.4, FlashAttention): a workgroup owns a
// block of query rows and streams key/value blocks through LDS; per block it
// forms the scores on chip, keeps a running row max and row sum, rescales
// the output accumulator when the max moves, adds exp(S - m) V, and divides
// by the sum once at the end.
//
// Why a kernel of its own: at d = 256 a wave that owns 32 query rows needs
// 128 accumulator registers for O alone, so only one such wave fits per SIMD
// and nothing overlaps its waits for the K/V copies and the stage barrier.
// Here a wave owns 16 query rows on the 16x16x32 MFMA (O takes 64
// registers), so two waves share each SIMD:
//   - 512 threads = 8 waves x 16 rows = 128 query rows per workgroup; K and V
//     stages of 64 keys (32 KiB each), double-buffered (128 KiB of LDS).
//   - Scores S^T = K Q^T in four 16-key tiles: K rows from LDS are the A
//     operand (lane = key row, 8 features), Q^T (registers) the B operand.
//     A lane then holds 4 keys of one query per tile; the 4 lanes c, c+16,
//     c+32, c+48 together hold a query's 64 keys.
//   - The rounded P of two consecutive tiles is directly the B operand of
//     O^T += V^T P^T over 32 keys (k-index 8g + j is key 4g + j for j < 4 and
//     16 + 4g + j - 4 otherwise; V^T is read in that order with the LDS
//     transpose read, so the sum is unchanged).
//   - LDS rows (512 bytes) are XOR-swizzled at 16-byte granularity: slot s of
//     row r is stored at s ^ sw(r), sw(r) = 2 ((r & 7) ^ ((r >> 1) & 4)) |
//     (r >> 3) & 1.  The K-operand read (16 consecutive rows, one slot each)
//     covers 16 distinct slots.  In the transpose read of V the 16-lane group
//     g addresses rows 4g .. 4g + 3 (and those + 16) of the same two slots;
//     the term (r >> 1) & 4 gives rows 8 apart (groups g and g + 2) disjoint
//     slot pairs, as it does rows 4 apart.  With sw(r) = 2 (r & 7) | (r >> 3) & 1
//     alone every transpose read took one extra pass (SQ_LDS_BANK_CONFLICT
//     68.2 M cycles per B4 H16 S4096 dispatch); with the term, 0.
//   - LDS reads are issued ahead of the MFMAs that consume them (K one
//     k-step, V^T four MFMAs), each MFMA with its reads one scheduling region.
//   - Softmax in base 2 with the scale folded into the exponent's FMA, lazy
//     rescaling (the reference max moves only when a block max exceeds it by
//     more than 2^8), P rounded to bf16 and summed from the rounded values.
//   - Causal tile pairing, longest-first order over ragged batches and the
//     XCD-grouped tile order follow prefill_bf16.hip.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kD = 256;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsW = 16;                    // query rows per wave
constexpr int kRows = kWaves * kRowsW;        // query rows per workgroup
constexpr int kKeys = 64;                     // keys per LDS stage and compute block
constexpr int kSlots = kD / 8;                // 16-byte slots per row
constexpr int kRowBytes = kD * 2;
constexpr int kStageBytes = kKeys * kRowBytes;
constexpr int KS = kD / 32;                   // k-steps of the score MFMA
constexpr int DT = kD / 16;                   // 16-feature output tiles
constexpr int kCopyBytes = kThreads * 16;     // one copy round of all waves
constexpr int kCopyRows = kCopyBytes / kRowBytes;
constexpr int kCopies = kStageBytes / kCopyBytes;
constexpr int kXcds = 8;
constexpr int kMaxRankB = 256;
constexpr float kRescaleSlack = 8.f;
constexpr float kLazyLimit = 256.f;
static_assert(kCopyRows % 16 == 0, "every copy round starts on the same swizzle phase");
// LDS reads in flight ahead of the MFMAs that consume them: K fragments one
// k-step (four MFMAs) ahead, V^T fragments four MFMAs ahead; each MFMA with
// the reads issued beside it is one scheduling region, so the distances hold
// (left to the scheduler, each P V MFMA waited on reads issued one MFMA
// earlier).  Measured for B4 H16 S4096: 0.647 -> 0.620 ms; deeper rings (two
// k-steps, six or eight MFMAs) were no faster.
constexpr int KPF = 1;
constexpr int VPF = 4;

__device__ __forceinline__ int sw(int r) { return (((r & 7) ^ ((r >> 1) & 4)) << 1) | ((r >> 3) & 1); }
// byte offset of (row, 16-byte slot) inside a swizzled stage
__device__ __forceinline__ uint32_t off(int row, int slot) {
  return (uint32_t)(row * kSlots + (slot ^ sw(row))) * 16u;
}

template <bool POS>
__global__ __launch_bounds__(kThreads, 1) void prefill_d256_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char k_s0[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char k_s1[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_s0[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_s1[kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qc = lane & 15;        // query column of this lane (MFMA column)
  const int grp = lane >> 4;       // 16-lane group: which 8 k-elements it feeds

  // Block -> (tile pair, head, batch), as in prefill_bf16.hip.
  const int n_qt = (p.Sq + kRows - 1) / kRows;
  const int G = p.Hq / p.Hkv;
  const int id = blockIdx.x;
  const bool pair = p.causal != 0 && p.pair != 0;
  const int n_pr = pair ? (n_qt + 1) / 2 : n_qt;
  int pr, h, b;
  if ((p.B * p.Hkv) % kXcds == 0) {
    const int xcd = id % kXcds, slot = id / kXcds;
    const int per_kv = G * n_pr;
    const int kvl = slot / per_kv, r = slot % per_kv;
    pr = r % n_pr;
    const int kv = kvl * kXcds + xcd;
    b = kv / p.Hkv;
    h = (kv % p.Hkv) * G + r / n_pr;
  } else {
    pr = id % n_pr;
    h = (id / n_pr) % p.Hq;
    b = id / (n_pr * p.Hq);
  }
  // Longest sequences first (ragged batches of at most kMaxRankB sequences).
  if ((p.kv_lens || p.cu_k) && p.B > 1 && p.B <= kMaxRankB) {
    int* keys = reinterpret_cast<int*>(v_s1);
    int* chosen = keys + kMaxRankB;
    if (tid < p.B) {
      int len;
      if (p.cu_k) {
        const int k0 = min(max(p.cu_k[tid], 0), p.total_k);
        const int k1 = min(max(p.cu_k[tid + 1], k0), p.total_k);
        len = min(k1 - k0, p.Skv);
      } else {
        len = min(max(p.kv_lens[tid], 0), p.Skv);
      }
      keys[tid] = len;
    }
    __syncthreads();
    if (tid < p.B) {
      const int mine = keys[tid];
      int rank = 0;
      for (int j = 0; j < p.B; ++j) {
        const int o = keys[j];
        rank += (o > mine || (o == mine && j < tid)) ? 1 : 0;
      }
      if (rank == b) *chosen = tid;
    }
    __syncthreads();
    b = *chosen;       // v_s1 is first written by stage 1's copies, after the first stage barrier
  }
  const int g = h / G;

  // This sequence's geometry (padded [B, H, S, d] or packed [total, H, d]).
  int sq, n;
  int64_t qs, kvs;
  const uint16_t *qp, *kp, *vp;
  uint16_t* op;
  if (p.cu_q) {
    const int q0 = min(max(p.cu_q[b], 0), p.total_q);
    const int q1 = min(max(p.cu_q[b + 1], q0), p.total_q);
    const int k0 = min(max(p.cu_k[b], 0), p.total_k);
    const int k1 = min(max(p.cu_k[b + 1], k0), p.total_k);
    sq = min(q1 - q0, p.Sq);
    n = min(k1 - k0, p.Skv);
    qs = (int64_t)p.Hq * kD;
    kvs = (int64_t)p.Hkv * kD;
    qp = static_cast<const uint16_t*>(p.q) + (int64_t)q0 * qs + (int64_t)h * kD;
    op = static_cast<uint16_t*>(p.o) + (int64_t)q0 * qs + (int64_t)h * kD;
    kp = static_cast<const uint16_t*>(p.k) + (int64_t)k0 * kvs + (int64_t)g * kD;
    vp = static_cast<const uint16_t*>(p.v) + (int64_t)k0 * kvs + (int64_t)g * kD;
  } else {
    sq = p.Sq;
    n = p.Skv;
    if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);
    qs = kD;
    kvs = kD;
    qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + h) * p.Sq * kD;
    op = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + h) * p.Sq * kD;
    kp = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.Hkv + g) * p.Skv * kD;
    vp = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.Hkv + g) * p.Skv * kD;
  }
  const int kv_row_bytes = (int)kvs * 2;
  const int n_qt_b = (sq + kRows - 1) / kRows;
  const int n_pr_b = pair ? (n_qt_b + 1) / 2 : n_qt_b;
  if (pr >= n_pr_b) return;         // uniform over the workgroup, before any further barrier

  // Staging: copy u of wave w fills LDS bytes u*kCopyBytes + w*1024 + 16*lane
  // of a stage, i.e. row st_row0 + u*kCopyRows, physical slot st_phys, and
  // fetches logical slot st_phys ^ sw(row) of that row (the same for every u).
  const int st_byte0 = wave * 1024 + lane * 16;
  const int st_row0 = st_byte0 / kRowBytes;
  const int st_slot = ((st_byte0 % kRowBytes) / 16) ^ sw(st_row0);
  const int kv_bytes = n > 0 ? (n - 1) * kv_row_bytes + kRowBytes : 0;
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(kp, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(vp, kv_bytes);
  const int wave_chunk = __builtin_amdgcn_readfirstlane(wave * 1024);
  auto copy_block = [&](__amdgpu_buffer_rsrc_t rsrc, unsigned char* dst, int j0) {
    unsigned char* d = dst + wave_chunk;
    if (j0 + kKeys <= n) {
#pragma unroll
      for (int u = 0; u < kCopies; ++u)
        buffer_to_lds16(rsrc, d + u * kCopyBytes, st_row0 * kv_row_bytes + st_slot * 16,
                        (j0 + u * kCopyRows) * kv_row_bytes);
    } else {
#pragma unroll
      for (int u = 0; u < kCopies; ++u) {
        const int row = st_row0 + u * kCopyRows;
        buffer_to_lds16(rsrc, d + u * kCopyBytes, min(j0 + row, n - 1) * kv_row_bytes + st_slot * 16, 0);
      }
    }
  };
  auto kbuf = [&](auto st_c) -> unsigned char* {
    if constexpr (decltype(st_c)::value == 0) return k_s0; else return k_s1;
  };
  auto vbuf = [&](auto st_c) -> unsigned char* {
    if constexpr (decltype(st_c)::value == 0) return v_s0; else return v_s1;
  };

  // Lane-constant LDS offsets.  K operand of k-step ks, tile kt: row
  // 16 kt + qc, slot 4 ks + grp (tile kt adds kt * 16 rows: sw repeats every
  // 16 rows).  V^T transpose reads of output tile t: group grp addresses rows
  // 4 grp + (lane & 15) / 4 (and those + 16), columns 16 t + 4 (lane & 3).
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = off(qc, 4 * ks + grp);
  const int vr0 = 4 * grp + (qc >> 2);
  uint32_t v_lo[DT], v_hi[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    const int c = 16 * t + 4 * (qc & 3);
    v_lo[t] = off(vr0, c >> 3) + (c & 7) * 2;
    v_hi[t] = off(vr0 + 16, c >> 3) + (c & 7) * 2;
  }

  const int n_pass = (pair && n_qt_b - 1 - pr != pr) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
  const int qt = pass == 0 ? n_qt_b - 1 - pr : pr;
  const int tile_row0 = qt * kRows;
  const int wave_row0 = tile_row0 + wave * kRowsW;
  const int my_row = wave_row0 + qc;
  const int last_row = min(tile_row0 + kRows, sq) - 1;
  const int diag = p.causal != 0 ? n - sq : n;
  const int kend = min(n, max(0, last_row + diag + 1));
  const int n_blocks = (kend + kKeys - 1) / kKeys;
  const int wave_last_row = min(wave_row0 + kRowsW - 1, sq - 1);
  const int my_last = my_row + diag;

  // Q^T as the B operand: lane (qc, grp) holds Q[my_row][32 ks + 8 grp .. +7].
  bf16x8 qreg[KS];
  {
    const int r = max(min(my_row, sq - 1), 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = as_bf16x8(ld16(qp + (int64_t)r * qs + 32 * ks + 8 * grp));
  }

  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{};
  float mref = kNegInf;
  float lsum = 0.f;
  const float c = p.scale_log2;
  constexpr float neutral = POS ? kNegInf : kPosInf;

  // S^T of a 64-key block: four 16-key tiles, K fragments read KPF k-steps ahead.
  auto scores = [&](auto st_c, f32x4 (&sacc)[4]) {
    const unsigned char* kb = kbuf(st_c);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x4{};
    u32x4 a[KPF + 1][4];
#pragma unroll
    for (int ks = 0; ks < KPF; ++ks)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) a[ks][kt] = *reinterpret_cast<const u32x4*>(kb + kt * 16 * kRowBytes + k_off[ks]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + KPF < KS) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          a[(ks + KPF) % (KPF + 1)][kt] = *reinterpret_cast<const u32x4*>(kb + kt * 16 * kRowBytes + k_off[ks + KPF]);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        sacc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[ks % (KPF + 1)][kt]), qreg[ks], sacc[kt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);     // keep the reads KPF k-steps ahead
    }
  };

  // Masking (blocks crossing the diagonal or the length only), the block
  // extreme and the lazy rescale.  Key of sacc[kt][i]: j0 + 16 kt + 4 grp + i.
  auto prepare = [&](auto masked_c, f32x4 (&sacc)[4], int j0) {
    constexpr bool MASKED = decltype(masked_c)::value;
    if (MASKED) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = j0 + 16 * kt + 4 * grp + i;
          if (j >= n || j > my_last) sacc[kt][i] = neutral;
        }
    }
    float traw = sacc[0][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) traw = POS ? fmaxf(traw, sacc[e / 4][e % 4]) : fminf(traw, sacc[e / 4][e % 4]);
    {
      const float o1 = shfl_xor(traw, 16);
      traw = POS ? fmaxf(traw, o1) : fminf(traw, o1);
      const float o2 = shfl_xor(traw, 32);
      traw = POS ? fmaxf(traw, o2) : fminf(traw, o2);
    }
    const float tmax = (MASKED && traw == neutral) ? kNegInf : traw * c;
    const float cand = fmaxf(mref, tmax);
    if (__builtin_expect(__any(cand > mref + kRescaleSlack), 0)) {
      const float alpha = cand == kNegInf ? 1.f : exp2_fast(mref - cand);
      mref = cand;
      lsum *= alpha;
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;
    }
  };

  // P = exp2(s c - m_ref) rounded to bf16: pb[kk] is the B operand of the
  // P V k-step over keys 32 kk .. 32 kk + 31 (tiles 2 kk and 2 kk + 1).
  // Returns this lane's sum of the rounded values.
  auto probabilities = [&](auto masked_c, const f32x4 (&sacc)[4], u32x4 (&pb)[2]) -> float {
    constexpr bool MASKED = decltype(masked_c)::value;
    const float negm = -mref;
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kt = 2 * kk + e / 2, i0 = 2 * (e % 2);
        const float s0 = sacc[kt][i0], s1 = sacc[kt][i0 + 1];
        float p0 = exp2_fast(fmaf(s0, c, negm));
        float p1 = exp2_fast(fmaf(s1, c, negm));
        if (MASKED) {
          p0 = s0 == neutral ? 0.f : p0;
          p1 = s1 == neutral ? 0.f : p1;
        }
        w[e] = pack_bf16x2(p0, p1);
        psum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[e]), kOnesBf16x2, psum, false);
      }
      pb[kk] = u32x4{w[0], w[1], w[2], w[3]};
    }
    return psum;
  };

  // O^T += V^T P^T; V^T from transpose reads of the row-major V stage,
  // issued VPF MFMAs ahead (a 16-cycle MFMA is far shorter than an LDS read).
  auto accumulate = [&](auto st_c, const u32x4 (&pb)[2]) {
    const unsigned char* vb = vbuf(st_c);
    constexpr int NM = 2 * DT;
    auto vread = [&](int m) {
      const int kk = m / DT, t = m % DT;
      const u32x2 lo = lds_read_tr16x4(vb + kk * 32 * kRowBytes + v_lo[t]);
      const u32x2 hi = lds_read_tr16x4(vb + kk * 32 * kRowBytes + v_hi[t]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 vf[VPF + 1];
#pragma unroll
    for (int m = 0; m < VPF; ++m) vf[m] = vread(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + VPF < NM) vf[(m + VPF) % (VPF + 1)] = vread(m + VPF);
      const int kk = m / DT, t = m % DT;
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[m % (VPF + 1)]), as_bf16x8(pb[kk]), oacc[t],
                                                        0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);   // keep the reads VPF MFMAs ahead
    }
  };

  auto active = [&](int blk) {
    return wave_row0 < sq && blk < n_blocks && blk * kKeys <= wave_last_row + diag;
  };
  auto needs_mask = [&](int blk) {
    const int j0 = blk * kKeys;
    return (j0 + kKeys > n) || (j0 + kKeys - 1 > wave_row0 + diag);
  };
  auto block = [&](auto st_c, int blk) {
    if (active(blk)) {
      f32x4 sc[4];
      u32x4 pb[2];
      scores(st_c, sc);
      if (!needs_mask(blk)) {
        // P against the current reference first; the block extreme is only
        // needed when some P may exceed 2^kRescaleSlack (or on a row's first
        // block, where the sum is +inf).
        float psum = probabilities(std::false_type{}, sc, pb);
        if (__builtin_expect(__any(!(psum <= kLazyLimit)), 0)) {
          const float m_old = mref;
          prepare(std::false_type{}, sc, blk * kKeys);
          if (__any(mref != m_old)) psum = probabilities(std::false_type{}, sc, pb);
        }
        lsum += psum;
      } else {
        prepare(std::true_type{}, sc, blk * kKeys);
        lsum += probabilities(std::true_type{}, sc, pb);
      }
      __builtin_amdgcn_sched_barrier(0);
      accumulate(st_c, pb);
    }
  };
  // One 64-key block per stage: the next stage's copies go to the other
  // buffer (last read in the previous stage, closed by its barrier) before
  // the block; one barrier closes the stage.
  auto stage_step = [&](auto st_c, int sb) {
    using Sn = std::integral_constant<int, 1 - decltype(st_c)::value>;
    if (sb + 1 < n_blocks) {
      copy_block(k_rsrc, kbuf(Sn{}), (sb + 1) * kKeys);
      copy_block(v_rsrc, vbuf(Sn{}), (sb + 1) * kKeys);
    }
    block(st_c, sb);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem();
    __syncthreads();
  };
  if (n_blocks > 0) {
    copy_block(k_rsrc, k_s0, 0);
    copy_block(v_rsrc, v_s0, 0);
  }
  wait_vmem();
  __syncthreads();
  for (int sb = 0; sb < n_blocks; sb += 2) {
    stage_step(std::integral_constant<int, 0>{}, sb);
    if (sb + 1 < n_blocks) stage_step(std::integral_constant<int, 1>{}, sb + 1);
  }

  // Epilogue: O = O_acc / l; lane (qc, grp) holds features 16 t + 4 grp .. +3.
  float l = lsum + shfl_xor(lsum, 16);
  l += shfl_xor(l, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (my_row < sq) {
    uint16_t* orow = op + (int64_t)my_row * qs;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const u32x2 w = {pack_bf16x2(oacc[t][0] * inv, oacc[t][1] * inv),
                       pack_bf16x2(oacc[t][2] * inv, oacc[t][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * t + 4 * grp) = w;
    }
  }
  }  // tile pass
}

}  // namespace

hipError_t launch_prefill_d256(const PrefillParams& p, hipStream_t stream) {
  const int n_qt = (p.Sq + kRows - 1) / kRows;
  const int n_pr = (p.causal && p.pair) ? (n_qt + 1) / 2 : n_qt;
  const dim3 grid((unsigned)n_pr * p.Hq * p.B);
  if (p.scale_log2 >= 0.f) hipLaunchKernelGGL((prefill_d256_kernel<true>), grid, dim3(kThreads), 0, stream, p);
  else hipLaunchKernelGGL((prefill_d256_kernel<false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace attn

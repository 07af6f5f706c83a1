// prefill_bf16.hip -- bf16 attention forward on gfx950 matrix cores.
//
// The tiled online-softmax loop of "GPU learning day 24: Operator Fusion",
// section 3.4 (FlashAttention): a workgroup owns a block of query rows and
// streams key/value blocks through LDS; per block it forms the scores on
// chip, keeps a running row max and row sum, rescales the output
// accumulator when the max moves, and adds exp(S - m) V.  One division at the
// end.  The score matrix never leaves the chip.
//
// gfx950 design
//   - 512 threads = 8 waves; each wave owns 32 query rows (256 per workgroup,
//     one workgroup per CU at d = 128).  At d = 256 (only the rotary
//     variants: d = 256 without rotation runs prefill_d256.hip): 256
//     threads, 4 waves (one per SIMD, so a wave may use 512 registers), 128
//     rows.  Large tiles halve the K/V traffic per query row against 128-row
//     tiles; with two waves per SIMD one wave's matrix work runs while the
//     other is in its softmax.
//   - Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K rows (from LDS) are the A operand and Q^T (held in registers for the
//     whole loop) is the B operand.  In the accumulator each lane then holds
//     one query column and 16 keys of it, so the row max and row sum are
//     lane-local apart from one exchange between the two lane halves.
//   - The same accumulator, rounded to bf16, is directly the B operand of
//     O^T += V^T P^T (the order of keys inside a 16-key step is permuted
//     consistently on both operands, which leaves the sum unchanged).
//   - V^T is read from the row-major V block in LDS with the LDS transpose
//     read (ds_read_b64_tr_b16), so V is never transposed in memory.
//   - K and V are staged through LDS 128 keys at a time, double-buffered
//     (128 KiB at d = 128), by buffer loads that write LDS directly; the
//     matrix work on a stage is done as two 64-key compute blocks, and the
//     copies of the next stage are issued between them (issuing them before
//     the first block measured slower); one barrier per stage.  Each copy's
//     LDS base and global offset are scalars, so a copy costs no vector ALU
//     work.  The loop is unrolled over the
//     two buffers and the two halves, so every LDS address is a lane
//     constant plus an immediate offset.
//   - In the score MFMAs the K fragments of k-step ks+1 are read while the
//     MFMAs of k-step ks run.
//   - LDS rows are XOR-swizzled at 16-byte granularity (Tile::sw) so the
//     row-parallel operand reads and the transpose reads are free of bank
//     conflicts.
//   - Softmax in base 2: the scale times log2(e) is folded into the FMA that
//     forms the exponent; the block max is taken on raw scores (v_max3).
//   - Lazy rescaling: the reference max of a row only moves when a block's
//     max exceeds it by more than 2^8, so the accumulator is rescaled on a
//     few blocks per row instead of every block.
//   - P is rounded to bf16 before P V and the running sum is accumulated
//     from the rounded values (v_dot2 with (1, 1)), so a constant V comes
//     back exactly.
//   - Masking code exists only on the path for blocks that cross the causal
//     diagonal or the length limit, and a wave skips the matrix work of a
//     block wholly above its rows.
//   - Causal: a workgroup processes the query tiles n_qt-1-p and p in turn,
//     so every workgroup has the same work; all pairs of one KV head are
//     consecutive on one XCD (workgroups go to XCD id % 8) and stream its K/V
//     through the same L2.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kKeys = 64;    // keys per compute block
// P V: V^T fragments read this many MFMAs ahead of the MFMA that consumes
// them, each MFMA with the reads issued beside it one scheduling region (the
// compiler's own placement left the first MFMAs of a block waiting on reads
// just issued).  Headline shape: 0.564 -> 0.551 ms; one ahead was slower,
// two about halfway.
constexpr int kVAhead = 3;
constexpr int kXcds = 8;                      // accelerator complex dies of an MI355X
constexpr int kMaxRankB = 256;                // longest-first order up to this many sequences
constexpr float kRescaleSlack = 8.f;   // base-2 headroom before the accumulator is rescaled
constexpr float kLazyLimit = 256.f;    // 2^kRescaleSlack: the largest P the lazy rescale allows
static_assert(kLazyLimit == 256.f && kRescaleSlack == 8.f, "kLazyLimit is 2^kRescaleSlack");

// Workgroup shape per head dimension.  d = 64, 128: 8 waves (two per SIMD),
// 256 query rows, 128-key LDS stages (two compute blocks).  d = 256: the
// output accumulator alone takes 128 registers per lane, so 4 waves (one per
// SIMD, up to 512 registers), 128 rows and 64-key stages.
template <int D>
struct Cfg {
  static constexpr int kThreads = D == 256 ? 256 : 512;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kRows = kWaves * 32;               // query rows per workgroup
  static constexpr int kStage = D == 256 ? 64 : 128;      // keys per LDS stage
  static constexpr int kBlocksPerStage = kStage / kKeys;
};

template <int D>
struct Tile {
  static constexpr int kStage = Cfg<D>::kStage;
  static constexpr int kSlots = D / 8;                    // 16-byte slots per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kStage * kRowBytes;       // one K or V stage
  static constexpr int kSubBytes = kKeys * kRowBytes;     // one compute block inside it
  static constexpr int kPiecesPerThread = kStage * kSlots / Cfg<D>::kThreads;
  // Swizzle of row r: its 16-byte slot s is stored at slot s ^ sw(r).  With
  // gfx950's 64 four-byte LDS banks (a row of 16 slots spans them all once)
  // two access patterns must hit distinct banks: the K-operand read (16
  // consecutive rows, one slot each: sw must permute 0..15 over 16 rows) and
  // the transpose read of V (4 rows aligned to 4, 4 consecutive slots each:
  // the rows' slot quads must not overlap).  For 8-slot rows (d = 64) two
  // rows share the 64 banks, so the same holds within even and odd rows.
  // 32-slot rows (d = 256) span the banks twice; slot s and s + 16 share
  // banks, and the 16-slot permutation (which never moves a slot across
  // that boundary) keeps both patterns conflict-free.
  __device__ static __forceinline__ int sw(int r) {
    if (kSlots >= 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // byte offset of (row, 16-byte slot) inside a swizzled block
  __device__ static __forceinline__ uint32_t off(int row, int slot) {
    return (uint32_t)(row * kSlots + (slot ^ sw(row))) * 16u;
  }
};

// One kernel serves causal and non-causal calls: the mask is a per-sequence
// offset (row i sees keys j <= i + diag; diag = n - S_q for the bottom-right
// causal mask, n for none), which compiles to fewer registers than separate
// non-causal instances (those spilled at d = 256 and ran 8-15% slower at
// d = 64 and 128).  POS: the scale is >= 0, so the block extreme of the raw
// scores is their max (a negative scale needs their min).  d = 64 is held
// to 128 registers so two workgroups share a CU (four waves per SIMD; its
// LDS stages take 64 KiB); the other variants run one workgroup per CU.
// ROPE: 0 none; 1 Q rows are rotated by the rotary table as they are loaded
// (K arrives rotated); 2 Q and every K stage are rotated.
template <int D, bool POS, int ROPE>
__global__ __launch_bounds__(Cfg<D>::kThreads, (D == 64 && ROPE < 2) ? 4 : 1) void prefill_bf16_kernel(PrefillParams p) {
  using T = Tile<D>;
  constexpr int kThreads = Cfg<D>::kThreads;
  constexpr int kRows = Cfg<D>::kRows;
  constexpr int kStage = Cfg<D>::kStage;
  constexpr int BPS = Cfg<D>::kBlocksPerStage;
  constexpr int KS = D / 16;       // k-steps of the score MFMA (16 features each)
  constexpr int DT = D / 32;       // 32-feature output tiles
  constexpr int NP = T::kPiecesPerThread;

  // Two stages of K and V, as separate arrays so the compiler can see that
  // filling one stage does not touch the stage being read.
  __shared__ __attribute__((aligned(16))) unsigned char k_s0[T::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char k_s1[T::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_s0[T::kBytes];
  __shared__ __attribute__((aligned(16))) unsigned char v_s1[T::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;      // which 8-feature half of a 16-step this lane feeds
  const int col = lane & 31;       // query column of this lane in the accumulators

  // Block -> (tile pair, head, batch).  Workgroups are dealt to the 8 XCDs
  // round-robin by id (id % 8); when the (batch, KV head) pairs divide
  // evenly over the XCDs, every workgroup of one KV head lands on the same
  // XCD, which then serves that KV head's K/V blocks from its own L2.
  const int n_qt = (p.Sq + kRows - 1) / kRows;
  const int G = p.Hq / p.Hkv;
  const int id = blockIdx.x;
  // Causal and paired: workgroup pair index pr covers tiles n_qt-1-pr then
  // pr (one tile when they coincide); causal unpaired: tile n_qt-1-pr
  // (heaviest first); non-causal: tile pr.
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
  // Longest sequences first: with per-sequence lengths (and at most
  // kMaxRankB sequences) the batch index decoded above is a rank, and the
  // workgroup takes the sequence with that many longer ones before it (ties
  // by index), so the lowest workgroup ids -- dispatched first -- take the
  // longest sequences.  Every workgroup computes the same order.  The
  // lengths pass through v_s1, which no copy writes before the first stage.
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
    b = *chosen;
  }
  const int g = h / G;

  // This sequence's geometry.  Padded layout [B, H, S, d]: rows of a head are
  // d apart, S_q query rows, kv_lens[b] (or S_kv) keys.  Packed layout
  // [total, H, d]: rows are H*d apart and the sequence's lengths come from
  // the offsets (clamped to the totals and the stated maxima).
  int sq, n;
  int64_t qs, kvs;                  // row strides of q/o and of k/v (elements)
  const uint16_t *qp, *kp, *vp;
  uint16_t* op;
  if (p.cu_q) {
    const int q0 = min(max(p.cu_q[b], 0), p.total_q);
    const int q1 = min(max(p.cu_q[b + 1], q0), p.total_q);
    const int k0 = min(max(p.cu_k[b], 0), p.total_k);
    const int k1 = min(max(p.cu_k[b + 1], k0), p.total_k);
    sq = min(q1 - q0, p.Sq);
    n = min(k1 - k0, p.Skv);
    qs = (int64_t)p.Hq * D;
    kvs = (int64_t)p.Hkv * D;
    qp = static_cast<const uint16_t*>(p.q) + (int64_t)q0 * qs + (int64_t)h * D;
    op = static_cast<uint16_t*>(p.o) + (int64_t)q0 * qs + (int64_t)h * D;
    kp = static_cast<const uint16_t*>(p.k) + (int64_t)k0 * kvs + (int64_t)g * D;
    vp = static_cast<const uint16_t*>(p.v) + (int64_t)k0 * kvs + (int64_t)g * D;
  } else {
    sq = p.Sq;
    n = p.Skv;
    if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);
    qs = D;
    kvs = D;
    qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + h) * p.Sq * D;
    op = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + h) * p.Sq * D;
    kp = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
    vp = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  }
  const int kv_row_bytes = (int)kvs * 2;
  // this sequence's own tiles (fewer than the grid's when it is shorter)
  const int n_qt_b = (sq + kRows - 1) / kRows;
  const int n_pr_b = pair ? (n_qt_b + 1) / 2 : n_qt_b;
  if (pr >= n_pr_b) return;         // uniform over the workgroup, before any barrier

  const int n_pass = (pair && n_qt_b - 1 - pr != pr) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
  const int qt = pass == 0 ? n_qt_b - 1 - pr : pr;   // unpaired: pass 0 only
  const int tile_row0 = qt * kRows;
  const int wave_row0 = tile_row0 + wave * 32;
  const int my_row = wave_row0 + col;
  const int last_row = min(tile_row0 + kRows, sq) - 1;
  // row i sees keys j <= i + diag: bottom-right causal, or every key
  const int diag = p.causal != 0 ? n - sq : n;
  const int kend = min(n, max(0, last_row + diag + 1));
  const int n_blocks = (kend + kKeys - 1) / kKeys;
  const int wave_last_row = min(wave_row0 + 31, sq - 1);
  const int my_last = my_row + diag;   // last key this row sees (>= n - 1 without a mask)

  // Q^T as the B operand: lane (col, half) holds Q[my_row][16*ks + 8*half .. +7].
  bf16x8 qreg[KS];
  {
    const int r = max(min(my_row, sq - 1), 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = as_bf16x8(ld16(qp + (int64_t)r * qs + 16 * ks + 8 * half));
    if constexpr (ROPE >= 1) {
      // this row's position (bottom-right aligned; rows that see no key use 0)
      const int pos = min(max(r + n - sq, 0), p.rope_rows - 1);
      const float* cs = p.rope + (int64_t)pos * D;
#pragma unroll
      for (int kp = 0; kp < KS / 2; ++kp) {   // features 16kp + 8half + e and their partners + d/2
        const float* c = cs + 16 * kp + 8 * half;
        u32x4 x1 = __builtin_bit_cast(u32x4, qreg[kp]), x2 = __builtin_bit_cast(u32x4, qreg[kp + KS / 2]);
        rope8(x1, x2, *reinterpret_cast<const f32x4*>(c), *reinterpret_cast<const f32x4*>(c + 4),
              *reinterpret_cast<const f32x4*>(c + D / 2), *reinterpret_cast<const f32x4*>(c + D / 2 + 4));
        qreg[kp] = as_bf16x8(x1);
        qreg[kp + KS / 2] = as_bf16x8(x2);
      }
    }
  }

  // Staging by direct global -> LDS copies.  Copy u of wave w fills the
  // 1 KiB LDS chunk c = u*kWaves + w of a stage; lane i lands at byte 16*i
  // of it, i.e. at (row, physical slot), and so fetches logical slot
  // physical ^ swizzle(row) of that row.  When the rows a copy round covers
  // are a multiple of 16 (d = 64, 128) the swizzle repeats from one copy to
  // the next and one lane offset serves all; otherwise (d = 256: 8 rows per
  // round) each copy has its own slot.
  constexpr int kPassBytes = kThreads * 16;                 // one copy round of all waves
  constexpr int kPassRows = kPassBytes / T::kRowBytes;      // key rows it covers
  constexpr bool kSameSlot = kPassRows % 16 == 0;
  const int st_byte0 = wave * 1024 + lane * 16;             // LDS byte of copy 0
  const int st_row0 = st_byte0 / T::kRowBytes;
  const int st_phys = (st_byte0 % T::kRowBytes) / 16;       // physical slot (same for every copy)
  int st_slot[kSameSlot ? 1 : NP];                          // logical slot of copy u
#pragma unroll
  for (int u = 0; u < (kSameSlot ? 1 : NP); ++u) st_slot[u] = st_phys ^ T::sw(st_row0 + u * kPassRows);
  auto slot_of = [&](int u) { return kSameSlot ? st_slot[0] : st_slot[u]; };
  uint32_t k_off[KS];                       // K operand (row col; row col+32 adds a constant)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = T::off(col, 2 * ks + half);
  uint32_t v_lo[DT], v_hi[DT];              // V^T transpose reads for k-step 0
  {
    const int grp = lane >> 4, src = lane & 15;
    const int r0 = 4 * (grp >> 1) + (src >> 2);
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const int cidx = 32 * t + 16 * (grp & 1) + 4 * (src & 3);
      v_lo[t] = T::off(r0, cidx >> 3) + (cidx & 7) * 2;
      v_hi[t] = T::off(r0 + 8, cidx >> 3) + (cidx & 7) * 2;
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float mref = kNegInf;   // reference max (base-2 units) of this lane's query
  float lsum = 0.f;       // this lane's share of the running sum
  const float c = p.scale_log2;
  constexpr float neutral = POS ? kNegInf : kPosInf;   // masked raw score

  auto kbuf = [&](auto stage_c) -> unsigned char* {
    if constexpr (decltype(stage_c)::value == 0) return k_s0; else return k_s1;
  };
  auto vbuf = [&](auto stage_c) -> unsigned char* {
    if constexpr (decltype(stage_c)::value == 0) return v_s0; else return v_s1;
  };

  // Copy one stage of K (or V) into LDS.  Rows past n are clamped
  // to row n-1 (only in the last stage) so no byte beyond a sequence is read.
  // one head's rows of this sequence: (n - 1) strides plus one row
  const int kv_bytes = n > 0 ? (n - 1) * kv_row_bytes + T::kRowBytes : 0;
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(kp, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(vp, kv_bytes);
  const int wave_chunk = __builtin_amdgcn_readfirstlane(wave * 1024);   // scalar LDS offset
  auto copy_block = [&](__amdgpu_buffer_rsrc_t rsrc, unsigned char* dst, int j0) {
    unsigned char* d = dst + wave_chunk;
    if (j0 + kStage <= n) {
#pragma unroll
      for (int u = 0; u < NP; ++u)
        buffer_to_lds16(rsrc, d + u * kPassBytes, st_row0 * kv_row_bytes + slot_of(u) * 16,
                        (j0 + u * kPassRows) * kv_row_bytes);
    } else {
#pragma unroll
      for (int u = 0; u < NP; ++u) {
        const int row = st_row0 + u * kPassRows;
        buffer_to_lds16(rsrc, d + u * kPassBytes, min(j0 + row, n - 1) * kv_row_bytes + slot_of(u) * 16, 0);
      }
    }
  };
  auto load_k = [&](auto stage_c, int j0) { copy_block(k_rsrc, kbuf(stage_c), j0); };
  auto load_v = [&](auto stage_c, int j0) { copy_block(v_rsrc, vbuf(stage_c), j0); };

  // Rotary embedding of a K stage, done once per workgroup in LDS: item
  // (row r, slot pair sl) rotates the 8 features of slot sl with their
  // partners in slot sl + kSlots/2 at position j0 + r.  The table rows are
  // fetched into registers when the stage's copies are issued and applied
  // after the stage has landed.
  constexpr int HS = T::kSlots / 2;
  constexpr int RIT = ROPE == 2 ? kStage * HS / kThreads : 1;   // items per thread per stage
  // d = 256 has no registers to hold the table rows across a block: they are
  // fetched after the stage has landed, two items at a time, just before
  // their rotation (rope_late).
  constexpr bool kLateFetch = D == 256;
  f32x4 rcs[kLateFetch ? 1 : RIT][4];
  auto rope_fetch = [&](int j0) {
#pragma unroll
    for (int i = 0; i < (kLateFetch ? 0 : RIT); ++i) {
      const int it = tid + i * kThreads, r = it / HS, sl = it % HS;
      const float* c = p.rope + (int64_t)min(j0 + r, p.rope_rows - 1) * D + 8 * sl;
      rcs[i][0] = *reinterpret_cast<const f32x4*>(c);
      rcs[i][1] = *reinterpret_cast<const f32x4*>(c + 4);
      rcs[i][2] = *reinterpret_cast<const f32x4*>(c + D / 2);
      rcs[i][3] = *reinterpret_cast<const f32x4*>(c + D / 2 + 4);
    }
  };
  auto rope_apply = [&](auto stage_c) {
    unsigned char* kb = kbuf(stage_c);
#pragma unroll
    for (int i = 0; i < (kLateFetch ? 0 : RIT); ++i) {
      const int it = tid + i * kThreads, r = it / HS, sl = it % HS;
      u32x4* a = reinterpret_cast<u32x4*>(kb + T::off(r, sl));
      u32x4* b = reinterpret_cast<u32x4*>(kb + T::off(r, sl + HS));
      u32x4 x1 = *a, x2 = *b;
      rope8(x1, x2, rcs[i][0], rcs[i][1], rcs[i][2], rcs[i][3]);
      *a = x1;
      *b = x2;
    }
  };
  auto rope_late = [&](auto stage_c, int j0) {
    unsigned char* kb = kbuf(stage_c);
#pragma unroll
    for (int i = 0; i < RIT; ++i) {
      const int it = tid + i * kThreads, r = it / HS, sl = it % HS;
      const float* c = p.rope + (int64_t)min(j0 + r, p.rope_rows - 1) * D + 8 * sl;
      u32x4* a = reinterpret_cast<u32x4*>(kb + T::off(r, sl));
      u32x4* b = reinterpret_cast<u32x4*>(kb + T::off(r, sl + HS));
      u32x4 x1 = *a, x2 = *b;
      rope8(x1, x2, *reinterpret_cast<const f32x4*>(c), *reinterpret_cast<const f32x4*>(c + 4),
            *reinterpret_cast<const f32x4*>(c + D / 2), *reinterpret_cast<const f32x4*>(c + D / 2 + 4));
      *a = x1;
      *b = x2;
      if (i % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // at most two items' table rows live
    }
  };

  // ---- the three phases of one key block --------------------------------
  // S^T = K Q^T for the two 32-key halves of compute block `sub` of an LDS
  // stage (the two accumulation chains are interleaved so consecutive MFMAs
  // are independent; the next k-step's K fragments are read meanwhile).
  auto scores = [&](auto stage_c, auto sub_c, f32x16 (&sacc)[2]) {
    const unsigned char* kb = kbuf(stage_c) + decltype(sub_c)::value * T::kSubBytes;
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    u32x4 a[2][2];   // K fragments: [k-step parity][32-key half]
    a[0][0] = *reinterpret_cast<const u32x4*>(kb + k_off[0]);
    a[0][1] = *reinterpret_cast<const u32x4*>(kb + 32 * T::kRowBytes + k_off[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
        a[(ks + 1) & 1][0] = *reinterpret_cast<const u32x4*>(kb + k_off[ks + 1]);
        a[(ks + 1) & 1][1] = *reinterpret_cast<const u32x4*>(kb + 32 * T::kRowBytes + k_off[ks + 1]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
        sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[ks & 1][sub]), qreg[ks], sacc[sub], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };

  // Masking (only for blocks that cross the diagonal or the length limit),
  // block extreme of the raw scores (max for a non-negative scale, min for a
  // negative one) and the lazy rescale of the accumulators.
  auto prepare = [&](auto masked_c, f32x16 (&sacc)[2], int j0) {
    constexpr bool MASKED = decltype(masked_c)::value;
    if (MASKED) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = j0 + 32 * sub + 8 * (i / 4) + 4 * half + (i % 4);
          if (j >= n || j > my_last) sacc[sub][i] = neutral;
        }
    }
    float traw = sacc[0][0];
    if (POS) {
#pragma unroll
      for (int i = 1; i < 32; ++i) traw = fmaxf(traw, sacc[i / 16][i % 16]);
      traw = max_across_halves(traw);
    } else {
#pragma unroll
      for (int i = 1; i < 32; ++i) traw = fminf(traw, sacc[i / 16][i % 16]);
      traw = min_across_halves(traw);
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

  // P = exp2(s*c - m_ref) rounded to bf16 (the B operand of P V); returns
  // this lane's sum of the rounded values (dot2 with (1, 1)).
  auto probabilities = [&](auto masked_c, const f32x16 (&sacc)[2], u32x4 (&pb)[4]) -> float {
    constexpr bool MASKED = decltype(masked_c)::value;
    const float negm = -mref;
    float psum = 0.f;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i0 = 8 * (cc % 2) + 2 * e;
        const float s0 = sacc[cc / 2][i0], s1 = sacc[cc / 2][i0 + 1];
        float p0 = exp2_fast(fmaf(s0, c, negm));
        float p1 = exp2_fast(fmaf(s1, c, negm));
        if (MASKED) {
          p0 = s0 == neutral ? 0.f : p0;
          p1 = s1 == neutral ? 0.f : p1;
        }
        w[e] = pack_bf16x2(p0, p1);
        psum = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(w[e]), kOnesBf16x2, psum, false);
      }
      pb[cc] = u32x4{w[0], w[1], w[2], w[3]};
    }
    return psum;
  };

  // O^T += V^T P^T from LDS stage S; V^T comes from transpose reads of the
  // row-major block (k-step outer, output tile inner: DT independent chains).
  constexpr int PF = kVAhead;
  auto vread = [&](auto stage_c, auto sub_c, int m) {
    const unsigned char* vb = vbuf(stage_c) + decltype(sub_c)::value * T::kSubBytes;
    const int cc = m / DT, t = m % DT;
    const u32x2 lo = lds_read_tr16x4(vb + cc * 16 * T::kRowBytes + v_lo[t]);
    const u32x2 hi = lds_read_tr16x4(vb + cc * 16 * T::kRowBytes + v_hi[t]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // The first PF fragments.  At d = 128 and 256 they are read before the
  // softmax, whose vector work then covers their latency (headline shape
  // 0.559 -> 0.551 ms, non-causal 0.994 -> 0.974); at d = 64, held to 128
  // registers, that would spill, so there they are read at the start of P V
  // (so too with K rotated in the kernel, which holds the table rows).
  constexpr bool kEarlyV = D != 64 && ROPE != 2;
  auto v_first = [&](auto stage_c, auto sub_c, u32x4 (&vf)[PF + 1]) {
#pragma unroll
    for (int m = 0; m < PF; ++m) vf[m] = vread(stage_c, sub_c, m);
  };
  auto accumulate = [&](auto stage_c, auto sub_c, const u32x4 (&pb)[4], u32x4 (&vf)[PF + 1]) {
    constexpr int NM = 4 * DT;
    if constexpr (!kEarlyV) v_first(stage_c, sub_c, vf);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + PF < NM) vf[(m + PF) % (PF + 1)] = vread(stage_c, sub_c, m + PF);
      const int cc = m / DT, t = m % DT;
      oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf[m % (PF + 1)]), as_bf16x8(pb[cc]), oacc[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Does any row of this wave see a key of block blk?  (wave-uniform; once
  // false it stays false for later blocks.)  A wave whose rows all lie past
  // the sequence's end (in a partial last tile) computes nothing; it still
  // takes part in the copies and barriers.
  auto active = [&](int blk) {
    return wave_row0 < sq && blk < n_blocks && blk * kKeys <= wave_last_row + diag;
  };
  auto needs_mask = [&](int blk) {
    const int j0 = blk * kKeys;
    return (j0 + kKeys > n) || (j0 + kKeys - 1 > wave_row0 + diag);
  };

  // ---- the key loop ------------------------------------------------------
  // An LDS stage holds BPS 64-key compute blocks.  The copies of the next
  // stage go to the other buffer, last read in the previous stage (closed by
  // its barrier): with two blocks per stage they are issued between them,
  // with one block before it.  One barrier closes the stage.
  const int n_stages = (n_blocks + BPS - 1) / BPS;
  auto block = [&](auto st_c, auto sub_c, int blk) {
    if (active(blk)) {
      f32x16 sc[2];
      u32x4 pb[4];
      u32x4 vf[PF + 1];
      scores(st_c, sub_c, sc);
      if constexpr (kEarlyV) {
        v_first(st_c, sub_c, vf);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (!needs_mask(blk)) {
        // P against the current reference first: the rescale is due only if
        // some P exceeds 2^kRescaleSlack, and then this lane's sum of P does
        // too (or is +inf on a row's first block), so the block extreme is
        // only computed on that rare path.  The result is the one prepare +
        // probabilities would give.
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
      accumulate(st_c, sub_c, pb, vf);
    }
  };
  auto stage_step = [&](auto st_c, int sb) {
    using Sn = std::integral_constant<int, 1 - decltype(st_c)::value>;
    const bool more = sb + 1 < n_stages;
    if constexpr (BPS == 1) {
      if (more) {
        load_k(Sn{}, (sb + 1) * kStage);
        load_v(Sn{}, (sb + 1) * kStage);
        if constexpr (ROPE == 2 && !kLateFetch) rope_fetch((sb + 1) * kStage);
      }
      block(st_c, std::integral_constant<int, 0>{}, sb);
    } else {
      block(st_c, std::integral_constant<int, 0>{}, 2 * sb);
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        load_k(Sn{}, (sb + 1) * kStage);
        load_v(Sn{}, (sb + 1) * kStage);
        if constexpr (ROPE == 2 && !kLateFetch) rope_fetch((sb + 1) * kStage);
      }
      if (2 * sb + 1 < n_blocks) block(st_c, std::integral_constant<int, 1>{}, 2 * sb + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem();
    __syncthreads();
    if constexpr (ROPE == 2) {
      if (more) {             // the next stage has landed: rotate its keys
        if constexpr (kLateFetch) rope_late(Sn{}, (sb + 1) * kStage); else rope_apply(Sn{});
        __syncthreads();
      }
    }
  };
  if (n_stages > 0) {
    load_k(std::integral_constant<int, 0>{}, 0);
    load_v(std::integral_constant<int, 0>{}, 0);
    if constexpr (ROPE == 2 && !kLateFetch) rope_fetch(0);
  }
  wait_vmem();
  __syncthreads();
  if constexpr (ROPE == 2) {
    if (n_stages > 0) {
      if constexpr (kLateFetch) rope_late(std::integral_constant<int, 0>{}, 0);
      else rope_apply(std::integral_constant<int, 0>{});
      __syncthreads();
    }
  }
  for (int sb = 0; sb < n_stages; sb += 2) {
    stage_step(std::integral_constant<int, 0>{}, sb);
    if (sb + 1 < n_stages) stage_step(std::integral_constant<int, 1>{}, sb + 1);
  }

  // Epilogue: O = O_acc / l, rounded to bf16.
  const float l = sum_across_halves(lsum);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (my_row < sq) {
    uint16_t* orow = op + (int64_t)my_row * qs;
#pragma unroll
    for (int t = 0; t < DT; ++t) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * t + 8 * q4 + 4 * half;
        u32x2 w = {pack_bf16x2(oacc[t][4 * q4] * inv, oacc[t][4 * q4 + 1] * inv),
                   pack_bf16x2(oacc[t][4 * q4 + 2] * inv, oacc[t][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = w;
      }
    }
  }
  }  // tile pass

}

template <int D>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  const int n_qt = (p.Sq + Cfg<D>::kRows - 1) / Cfg<D>::kRows;
  const int n_pr = (p.causal && p.pair) ? (n_qt + 1) / 2 : n_qt;
  dim3 grid((unsigned)n_pr * p.Hq * p.B);
  const dim3 block(Cfg<D>::kThreads);
  const bool pos = p.scale_log2 >= 0.f;
  if (p.rope && p.rope_k) {
    if (pos) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, 2>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, 2>), grid, block, 0, stream, p);
  } else if (p.rope) {
    if (pos) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, 1>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, 1>), grid, block, 0, stream, p);
  } else {
    if (pos) hipLaunchKernelGGL((prefill_bf16_kernel<D, true, 0>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((prefill_bf16_kernel<D, false, 0>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  if (p.d == 64) return launch<64>(p, stream);
  // d = 256 without the rotary embedding: 16-row waves, two per SIMD
  if (p.d == 256) return p.rope ? launch<256>(p, stream) : launch_prefill_d256(p, stream);
  return launch<128>(p, stream);
}

}  // namespace attn

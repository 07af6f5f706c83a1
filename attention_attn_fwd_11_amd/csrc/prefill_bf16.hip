// prefill_bf16.hip -- bf16 attention forward on gfx950 matrix cores.
//
// The tiled online-softmax loop of "GPU learning day 24: Operator Fusion",
// section 3.4 (FlashAttention): a workgroup owns a block of query rows and
// streams key/value blocks through LDS; per block it forms the scores on
// chip, raises the running row max, rescales the running sum and the output
// accumulator by exp(m_old - m_new), and adds exp(S - m_new) V.  One
// division at the end.  The score matrix never leaves the chip.
//
// gfx950 design
//   - 256 threads = 4 waves; each wave owns 32 query rows (128 per workgroup).
//   - Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     K rows (from LDS) are the A operand and Q^T (held in registers for the
//     whole loop) is the B operand.  In the accumulator each lane then holds
//     one query column and 16 keys of it, so the row max and row sum are
//     mostly lane-local; the two lane halves are joined with one exchange.
//   - The same accumulator, rounded to bf16, is directly the B operand of
//     O^T += V^T P^T (the order of keys inside a 16-key step is permuted
//     consistently on both operands, which leaves the sum unchanged).
//   - V^T is read from the row-major V block in LDS with the LDS transpose
//     read (ds_read_b64_tr_b16), so V is never transposed in memory.
//   - K/V blocks of 64 keys are double-buffered in LDS: the next block's
//     global loads are issued before the current block's matrix work and
//     written to the other buffer after it; one barrier per block.
//   - LDS rows are XOR-swizzled at 16-byte granularity so the row-parallel
//     operand reads and the transpose reads are free of bank conflicts.
//   - exp2 with log2(e) folded into the scale; P is rounded to bf16 before
//     P V and the running sum is accumulated from the rounded values, so a
//     constant V comes back exactly.
//   - Causal tiles are launched heaviest first; a wave skips the matrix work
//     of a block that lies wholly above its rows' diagonal, and masking is
//     applied only on blocks that cross the diagonal or the length limit.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kRows = 128;   // query rows per workgroup
constexpr int kKeys = 64;    // keys per LDS block
constexpr int kThreads = 256;

template <int D>
struct Tile {
  static constexpr int kSlots = D / 8;                    // 16-byte slots per row
  static constexpr int kBytes = kKeys * D * 2;            // one K or V block
  static constexpr int kPiecesPerThread = kKeys * kSlots / kThreads;
  // byte offset of (row, 16-byte slot) inside a swizzled block
  __device__ static __forceinline__ int off(int row, int slot) {
    return (row * kSlots + (slot ^ (row % kSlots))) * 16;
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(PrefillParams p) {
  using T = Tile<D>;
  constexpr int KS = D / 16;       // k-steps of the score MFMA (16 features each)
  constexpr int DT = D / 32;       // 32-feature output tiles
  constexpr int NP = T::kPiecesPerThread;

  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * 2 * T::kBytes];
  // stage s: K block at smem + s*kBytes, V block at smem + (2+s)*kBytes
  auto kbuf = [&](int stage) { return smem + stage * T::kBytes; };
  auto vbuf = [&](int stage) { return smem + (2 + stage) * T::kBytes; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;      // which 8-feature half of a 16-step this lane feeds
  const int col = lane & 31;       // query column of this lane in the accumulators

  // Block -> (query tile, head, batch).  Causal: heaviest (last) tiles first.
  const int n_qt = (p.Sq + kRows - 1) / kRows;
  const int per_tile = p.Hq * p.B;
  const int id = blockIdx.x;
  int qt = id / per_tile;
  if (CAUSAL) qt = n_qt - 1 - qt;
  const int h = (id % per_tile) % p.Hq;
  const int b = (id % per_tile) / p.Hq;
  const int g = h / (p.Hq / p.Hkv);

  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);

  const uint16_t* qp = static_cast<const uint16_t*>(p.q) + ((int64_t)b * p.Hq + h) * p.Sq * D;
  const uint16_t* kp = static_cast<const uint16_t*>(p.k) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  const uint16_t* vp = static_cast<const uint16_t*>(p.v) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  uint16_t* op = static_cast<uint16_t*>(p.o) + ((int64_t)b * p.Hq + h) * p.Sq * D;

  const int tile_row0 = qt * kRows;
  const int wave_row0 = tile_row0 + wave * 32;
  const int my_row = wave_row0 + col;
  const int last_row = min(tile_row0 + kRows, p.Sq) - 1;
  int kend = n;
  if (CAUSAL) kend = min(n, max(0, last_row + n - p.Sq + 1));
  const int n_blocks = (kend + kKeys - 1) / kKeys;

  // Q^T as the B operand: lane (col, half) holds Q[my_row][16*ks + 8*half .. +7].
  bf16x8 qreg[KS];
  {
    const int r = min(my_row, p.Sq - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qreg[ks] = as_bf16x8(ld16(qp + (int64_t)r * D + 16 * ks + 8 * half));
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  float m = kNegInf;      // running max (base-2 units) of this lane's query
  float lsum = 0.f;       // this lane's share of the running sum

  // Global -> register staging of one K/V block (rows clamped to n-1).
  u32x4 kst[NP], vst[NP];
  auto load_block = [&](int j0) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int piece = u * kThreads + tid;
      const int row = piece / T::kSlots, slot = piece % T::kSlots;
      const int64_t src = (int64_t)min(j0 + row, n - 1) * D + slot * 8;
      kst[u] = ld16(kp + src);
      vst[u] = ld16(vp + src);
    }
  };
  auto store_block = [&](int stage) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int piece = u * kThreads + tid;
      const int row = piece / T::kSlots, slot = piece % T::kSlots;
      *reinterpret_cast<u32x4*>(kbuf(stage) + T::off(row, slot)) = kst[u];
      *reinterpret_cast<u32x4*>(vbuf(stage) + T::off(row, slot)) = vst[u];
    }
  };

  if (n_blocks > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();

  for (int blk = 0; blk < n_blocks; ++blk) {
    const int stage = blk & 1;
    const int j0 = blk * kKeys;
    const bool has_next = blk + 1 < n_blocks;
    if (has_next) load_block(j0 + kKeys);

    // Does any row of this wave see a key of this block?  (wave-uniform)
    const int wave_last_row = min(wave_row0 + 31, p.Sq - 1);
    const bool active = !CAUSAL || j0 <= wave_last_row + n - p.Sq;
    if (active) {
      const unsigned char* kb = kbuf(stage);
      const unsigned char* vb = vbuf(stage);

      // S^T = K Q^T for the two 32-key halves of the block.
      f32x16 sacc[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        sacc[sub] = f32x16{};
        const int krow = 32 * sub + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(kb + T::off(krow, 2 * ks + half)));
          sacc[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[sub], 0, 0, 0);
        }
      }

      // Scale to base-2 units and mask where the block crosses a limit.
      const int wave_first_row = wave_row0;
      const bool need_mask = (j0 + kKeys > n) ||
                             (CAUSAL && j0 + kKeys - 1 > wave_first_row + n - p.Sq);
      const int my_last = CAUSAL ? my_row + n - p.Sq : n - 1;
      float tmax = kNegInf;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float s = sacc[sub][i] * p.scale_log2;
          if (need_mask) {
            const int j = j0 + 32 * sub + 8 * (i / 4) + 4 * half + (i % 4);
            if (j >= n || j > my_last) s = kNegInf;
          }
          sacc[sub][i] = s;
          tmax = fmaxf(tmax, s);
        }
      }
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float m_new = fmaxf(m, tmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      m = m_new;

      // P = exp2(S - m), rounded to bf16; the running sum uses the rounded P.
      u32x4 pb[4];
      float psum = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i0 = 8 * (c % 2) + 2 * e;
          const float p0 = exp2_fast(sacc[c / 2][i0] - m_use);
          const float p1 = exp2_fast(sacc[c / 2][i0 + 1] - m_use);
          w[e] = pack_bf16x2(p0, p1);
          psum += bf16_lo(w[e]) + bf16_hi(w[e]);
        }
        pb[c] = u32x4{w[0], w[1], w[2], w[3]};
      }
      lsum = lsum * alpha + psum;
#pragma unroll
      for (int t = 0; t < DT; ++t) oacc[t] *= alpha;

      // O^T += V^T P^T; V^T comes from transpose reads of the row-major block.
      const int grp = lane >> 4;          // 16-lane group
      const int src = lane & 15;          // source lane within the group
      const int khalf = grp >> 1;         // = half
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int d0 = 32 * t + 16 * (grp & 1);
        const int cidx = d0 + 4 * (src & 3);           // column this lane addresses
        const int cslot = cidx >> 3, cbyte = (cidx & 7) * 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int r0 = 16 * c + 4 * khalf + (src >> 2);
          const int r1 = r0 + 8;
          const u32x2 lo = lds_read_tr16x4(vb + T::off(r0, cslot) + cbyte);
          const u32x2 hi = lds_read_tr16x4(vb + T::off(r1, cslot) + cbyte);
          const bf16x8 a = as_bf16x8(u32x4{lo[0], lo[1], hi[0], hi[1]});
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pb[c]), oacc[t], 0, 0, 0);
        }
      }
    }

    if (has_next) store_block(stage ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l, rounded to bf16.
  const float l = lsum + shfl_xor(lsum, 32);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (my_row < p.Sq) {
    uint16_t* orow = op + (int64_t)my_row * D;
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
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  const int n_qt = (p.Sq + kRows - 1) / kRows;
  dim3 grid((unsigned)n_qt * p.Hq * p.B);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace attn

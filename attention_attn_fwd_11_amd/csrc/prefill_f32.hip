// prefill_f32.hip -- fp32 attention forward (vector ALU path).
//
// Tiled online softmax as in "GPU learning day 24: Operator Fusion", section
// 3.4 (FlashAttention loop): each workgroup owns a tile of query rows,
// walks the key/value sequence in blocks staged in LDS, keeps a running row
// max m and row sum l per query, rescales its accumulator when m grows, and
// divides by l once at the end.  Everything is fp32; exponentials are taken
// base 2 with log2(e) folded into the scale.
//
// Mapping: 512 threads per workgroup, eight adjacent lanes per query row,
// each lane owning an eighth of the features.  A score is eight partial dot
// products (one per lane) added by three DPP lane moves, so every lane of
// the row holds the full score; P V then accumulates each lane's eighth of the
// output.  This path is bound by each lane's serial chain over the keys, not
// by bandwidth, and has two tile shapes:
//   - small grids: 8-row tiles, the eight waves forming eight key groups;
//     group k walks key blocks k, k+8, ... with its own running (m, l, o)
//     per row, and the eight states of a row are merged at the end by the
//     same rescaling identity (weights 2^(m_k - M)).  Eight times the
//     workgroups, and an eighth of the keys per chain (B1 H2 S128 d64:
//     28 us per call with one 64-row group, 11 us with 16 rows in four
//     groups, 9 us with this shape);
//   - grids of at least kF32LargeGrid 64-row tiles: 64-row tiles, one key
//     group, so K and V are re-read from cache once per 64 query rows.
// Keys and values pass through LDS in 16-byte loads; the 8 rows of a wave
// read the same key row (broadcast) and its eight pieces lie in distinct
// banks.  This path exists for fp32 inputs, where matrix cores give no
// benefit at fp32 accuracy.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kF32Parts = 8;                          // lanes per query row
constexpr int kF32Threads = 512;                      // 64 rows' worth of lanes
// Grids of at least this many 64-row tiles use them (one key group, the
// fewest K/V re-reads); smaller grids use 8-row tiles with 8 key groups,
// which put eight times the workgroups on the chip and split each row's keys
// eight ways.
constexpr int64_t kF32LargeGrid = 512;

// Lane move within each row of 16 lanes (DPP control CTRL), as a float.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 adjacent lanes of a query row (an aligned half-row) with
// DPP moves: swap neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm
// 2,3,0,1), then mirror the half-row (lane i with 7 - i, in the other quad).
// Every lane ends with ((a0+a1)+(a2+a3)) + ((a4+a5)+(a6+a7)) up to the
// order of each addition's operands: the sum a butterfly over lane masks 1,
// 2, 4 forms, without going through the LDS crossbar.
__device__ __forceinline__ float row8_sum(float a) {
  a += dpp_move<0xB1>(a);
  a += dpp_move<0x4E>(a);
  a += dpp_move<0x141>(a);
  return a;
}

template <int D, bool CAUSAL, int ROWS>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(PrefillParams p) {
  constexpr int GROUPS = kF32Threads / (ROWS * kF32Parts);   // key groups
  constexpr int GT = ROWS * kF32Parts;                // threads per key group
  constexpr int F = D / kF32Parts;                    // features per lane
  // keys per LDS block (8-row tiles: 4 KiB of K per block, and 8 keys at
  // d = 256 so the merge area fits the blocks)
  constexpr int KB = ROWS == 64 ? 32 : (D == 256 ? 8 : 1024 / D);
  // K and V blocks of every group; after the loop the same memory holds each
  // group's state per row for the merge: o[D], m, l and two floats of
  // padding, so every record starts 16-byte aligned.
  constexpr int kRec = D + 4;
  __shared__ __attribute__((aligned(16))) float kv_s[GROUPS][2][KB][D];
  static_assert(GROUPS == 1 || GROUPS * ROWS * kRec <= GROUPS * 2 * KB * D, "merge area must fit");
  float* mrg = &kv_s[0][0][0][0];
  auto mrg_at = [&](int gr, int row) { return mrg + (gr * ROWS + row) * kRec; };

  const int tid = threadIdx.x;
  const int grp = tid / GT;             // key group (wave-uniform)
  const int gt = tid % GT;
  const int r = gt / kF32Parts, part = gt % kF32Parts;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (p.Hq / p.Hkv);
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);

  const float* qp = static_cast<const float*>(p.q) + ((int64_t)b * p.Hq + h) * p.Sq * D;
  const float* kp = static_cast<const float*>(p.k) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  const float* vp = static_cast<const float*>(p.v) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  float* op = static_cast<float*>(p.o) + ((int64_t)b * p.Hq + h) * p.Sq * D;

  const int row0 = qt * ROWS;
  const int i = row0 + r;                             // this lane's query row
  const int last_row = min(row0 + ROWS, p.Sq) - 1;
  int kend = n;                                       // keys any row of the tile may see
  if (CAUSAL) kend = min(n, max(0, last_row + n - p.Sq + 1));
  const int my_last = CAUSAL ? i + n - p.Sq : n - 1;  // last key this row sees
  const int nblk = (kend + KB - 1) / KB;
  const int iters = (nblk + GROUPS - 1) / GROUPS;   // the same for every group

  // this lane's eighth of its query row (zero past S_q)
  float q[F];
#pragma unroll
  for (int c = 0; c < F; c += 4) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
    if (i < p.Sq) w = *reinterpret_cast<const f32x4*>(qp + (int64_t)i * D + part * F + c);
    q[c] = w[0]; q[c + 1] = w[1]; q[c + 2] = w[2]; q[c + 3] = w[3];
  }

  float m = kNegInf, l = 0.f;
  float acc[F];
#pragma unroll
  for (int c = 0; c < F; ++c) acc[c] = 0.f;

  for (int it = 0; it < iters; ++it) {
    const int j0 = (it * GROUPS + grp) * KB;
    const bool has = j0 < kend;                       // uniform across the group
    __syncthreads();
    if (has) {
      for (int e = gt; e < KB * D / 4; e += GT) {
        const int rr = e / (D / 4), c4 = 4 * (e % (D / 4));
        const int64_t row = min(j0 + rr, n - 1);      // clamp: masked rows read a valid row
        *reinterpret_cast<f32x4*>(&kv_s[grp][0][rr][c4]) = *reinterpret_cast<const f32x4*>(kp + row * D + c4);
        *reinterpret_cast<f32x4*>(&kv_s[grp][1][rr][c4]) = *reinterpret_cast<const f32x4*>(vp + row * D + c4);
      }
    }
    __syncthreads();
    if (!has) continue;

    float s[KB];
#pragma unroll
    for (int rr = 0; rr < KB; ++rr) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < F; c += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&kv_s[grp][0][rr][part * F + c]);
        a = fmaf(q[c], kv[0], a);
        a = fmaf(q[c + 1], kv[1], a);
        a = fmaf(q[c + 2], kv[2], a);
        a = fmaf(q[c + 3], kv[3], a);
      }
      s[rr] = row8_sum(a);   // the row's 8 lanes are adjacent and aligned
    }
    float mt = kNegInf;
#pragma unroll
    for (int rr = 0; rr < KB; ++rr) {
      const int j = j0 + rr;
      const bool vis = j < n && j <= my_last;
      s[rr] = vis ? s[rr] * p.scale_log2 : kNegInf;
      mt = fmaxf(mt, s[rr]);
    }
    const float m_new = fmaxf(m, mt);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    l *= alpha;
#pragma unroll
    for (int rr = 0; rr < KB; ++rr) {
      s[rr] = exp2_fast(s[rr] - m_use);
      l += s[rr];
    }
#pragma unroll
    for (int c = 0; c < F; c += 4) {
      float a0 = acc[c] * alpha, a1 = acc[c + 1] * alpha, a2 = acc[c + 2] * alpha, a3 = acc[c + 3] * alpha;
#pragma unroll
      for (int rr = 0; rr < KB; ++rr) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(&kv_s[grp][1][rr][part * F + c]);
        a0 = fmaf(s[rr], vv[0], a0);
        a1 = fmaf(s[rr], vv[1], a1);
        a2 = fmaf(s[rr], vv[2], a2);
        a3 = fmaf(s[rr], vv[3], a3);
      }
      acc[c] = a0; acc[c + 1] = a1; acc[c + 2] = a2; acc[c + 3] = a3;
    }
    m = m_new;
  }

  if constexpr (GROUPS == 1) {
    if (i < p.Sq) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int c = 0; c < F; c += 4) {
        f32x4 w = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
        *reinterpret_cast<f32x4*>(op + (int64_t)i * D + part * F + c) = w;
      }
    }
    return;
  } else {
    // Merge the key groups' states of each row: M = max_k m_k, weights
    // 2^(m_k - M) (0 for a group that saw no key of the row), O = sum w_k o_k /
    // sum w_k l_k; a row that sees no key gets zeros.
    __syncthreads();                                    // every group is done with its blocks
    {
      float* st = mrg_at(grp, r);
#pragma unroll
      for (int c = 0; c < F; c += 4)
        *reinterpret_cast<f32x4*>(st + part * F + c) = f32x4{acc[c], acc[c + 1], acc[c + 2], acc[c + 3]};
      if (part == 0) {
        st[D] = m;
        st[D + 1] = l;
      }
    }
    __syncthreads();
    if (grp == 0 && i < p.Sq) {
      float M = kNegInf;
#pragma unroll
      for (int k = 0; k < GROUPS; ++k) M = fmaxf(M, mrg_at(k, r)[D]);
      float L = 0.f;
      float o[F];
#pragma unroll
      for (int c = 0; c < F; ++c) o[c] = 0.f;
      if (M != kNegInf) {
#pragma unroll
        for (int k = 0; k < GROUPS; ++k) {
          const float* st = mrg_at(k, r);
          const float w = st[D] == kNegInf ? 0.f : exp2_fast(st[D] - M);
          L += w * st[D + 1];
#pragma unroll
          for (int c = 0; c < F; ++c) o[c] = fmaf(w, st[part * F + c], o[c]);
        }
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
      for (int c = 0; c < F; c += 4) {
        f32x4 w = {o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
        *reinterpret_cast<f32x4*>(op + (int64_t)i * D + part * F + c) = w;
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  const int64_t tiles64 = (int64_t)((p.Sq + 63) / 64) * p.Hq * p.B;
  if (tiles64 >= kF32LargeGrid) {
    dim3 grid((p.Sq + 63) / 64, p.Hq, p.B);
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, 64>), grid, dim3(kF32Threads), 0, stream, p);
  } else {
    dim3 grid((p.Sq + 7) / 8, p.Hq, p.B);
    hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL, 8>), grid, dim3(kF32Threads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  if (p.d == 256) return p.causal ? launch<256, true>(p, stream) : launch<256, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace attn

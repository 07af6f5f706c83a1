// prefill_f32.hip -- fp32 attention forward (vector ALU path).
//
// Tiled online softmax as in "GPU learning day 24: Operator Fusion", section
// 3.4 (FlashAttention loop): each workgroup owns 64 query rows, walks the
// key/value sequence in 32-key blocks staged in LDS, keeps a running row max
// m and row sum l per query, rescales its accumulator when m grows, and
// divides by l once at the end.  Everything is fp32; exponentials are taken
// base 2 with log2(e) folded into the scale.
//
// Mapping: 512 threads per workgroup, eight adjacent lanes per query row;
// each lane owns an eighth of the features.  A score is eight partial dot
// products (one per lane) added by three exchanges, so every lane of the row
// holds the full score; P V then accumulates each lane's eighth of the
// output.  Spreading a row over lanes shortens each lane's serial chain,
// which bounds this latency-bound path (one lane per row: 70 us for
// B1 H2 S128 d64; four lanes: 45; eight: 28; sixteen: 35).  Keys and values
// pass through LDS in 32-key blocks (16-byte loads); the 8 rows of a wave
// read the same key row (broadcast) and its eight pieces lie in distinct
// banks.  This path exists for fp32 inputs, where matrix cores give no
// benefit at fp32 accuracy.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kF32Rows = 64;                      // query rows per workgroup
constexpr int kF32Keys = 32;                      // keys per LDS block
constexpr int kF32Parts = 8;                      // lanes per query row
constexpr int kF32Threads = kF32Rows * kF32Parts;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(PrefillParams p) {
  constexpr int F = D / kF32Parts;                // features per lane
  __shared__ __attribute__((aligned(16))) float k_s[kF32Keys][D];
  __shared__ __attribute__((aligned(16))) float v_s[kF32Keys][D];

  const int tid = threadIdx.x;
  const int r = tid / kF32Parts, part = tid % kF32Parts;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (p.Hq / p.Hkv);
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);

  const float* qp = static_cast<const float*>(p.q) + ((int64_t)b * p.Hq + h) * p.Sq * D;
  const float* kp = static_cast<const float*>(p.k) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  const float* vp = static_cast<const float*>(p.v) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  float* op = static_cast<float*>(p.o) + ((int64_t)b * p.Hq + h) * p.Sq * D;

  const int row0 = qt * kF32Rows;
  const int i = row0 + r;                          // this lane's query row
  const int last_row = min(row0 + kF32Rows, p.Sq) - 1;
  int kend = n;                                    // keys any row of the tile may see
  if (CAUSAL) kend = min(n, max(0, last_row + n - p.Sq + 1));
  const int my_last = CAUSAL ? i + n - p.Sq : n - 1;  // last key this row sees

  // this lane's quarter of its query row (zero past S_q)
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

  for (int j0 = 0; j0 < kend; j0 += kF32Keys) {
    __syncthreads();
    for (int e = tid; e < kF32Keys * D / 4; e += kF32Threads) {
      const int rr = e / (D / 4), c4 = 4 * (e % (D / 4));
      const int64_t row = min(j0 + rr, n - 1);       // clamp: masked rows read a valid row
      *reinterpret_cast<f32x4*>(&k_s[rr][c4]) = *reinterpret_cast<const f32x4*>(kp + row * D + c4);
      *reinterpret_cast<f32x4*>(&v_s[rr][c4]) = *reinterpret_cast<const f32x4*>(vp + row * D + c4);
    }
    __syncthreads();

    float s[kF32Keys];
#pragma unroll
    for (int rr = 0; rr < kF32Keys; ++rr) {
      float a = 0.f;
#pragma unroll
      for (int c = 0; c < F; c += 4) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&k_s[rr][part * F + c]);
        a = fmaf(q[c], kv[0], a);
        a = fmaf(q[c + 1], kv[1], a);
        a = fmaf(q[c + 2], kv[2], a);
        a = fmaf(q[c + 3], kv[3], a);
      }
#pragma unroll
      for (int msk = 1; msk < kF32Parts; msk <<= 1) a += shfl_xor(a, msk);   // the row's lanes are adjacent
      s[rr] = a;
    }
    float mt = kNegInf;
#pragma unroll
    for (int rr = 0; rr < kF32Keys; ++rr) {
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
    for (int rr = 0; rr < kF32Keys; ++rr) {
      s[rr] = exp2_fast(s[rr] - m_use);
      l += s[rr];
    }
#pragma unroll
    for (int c = 0; c < F; c += 4) {
      float a0 = acc[c] * alpha, a1 = acc[c + 1] * alpha, a2 = acc[c + 2] * alpha, a3 = acc[c + 3] * alpha;
#pragma unroll
      for (int rr = 0; rr < kF32Keys; ++rr) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(&v_s[rr][part * F + c]);
        a0 = fmaf(s[rr], vv[0], a0);
        a1 = fmaf(s[rr], vv[1], a1);
        a2 = fmaf(s[rr], vv[2], a2);
        a3 = fmaf(s[rr], vv[3], a3);
      }
      acc[c] = a0; acc[c + 1] = a1; acc[c + 2] = a2; acc[c + 3] = a3;
    }
    m = m_new;
  }

  if (i < p.Sq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < F; c += 4) {
      f32x4 w = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
      *reinterpret_cast<f32x4*>(op + (int64_t)i * D + part * F + c) = w;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  dim3 grid((p.Sq + kF32Rows - 1) / kF32Rows, p.Hq, p.B);
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), grid, dim3(kF32Threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace attn

// prefill_f32.hip -- fp32 attention forward (vector ALU path).
//
// Tiled online softmax as in "GPU learning day 24: Operator Fusion", section
// 3.4 (FlashAttention loop): each workgroup owns 64 query rows, walks the
// key/value sequence in 32-key blocks staged in LDS, keeps a running row max
// m and row sum l per query, rescales its accumulator when m grows, and
// divides by l once at the end.  Everything is fp32; exponentials are taken
// base 2 with log2(e) folded into the scale.
//
// Mapping: one wave per workgroup, one lane per query row.  The query tile
// sits in LDS (padded rows, conflict-free); keys and values are read from LDS
// as wave-wide broadcasts.  This path exists for fp32 inputs, where matrix
// cores give no benefit at fp32 accuracy.
#include "common.hpp"
#include "kernels.hpp"

namespace attn {

namespace {

constexpr int kF32Rows = 64;   // query rows per workgroup
constexpr int kF32Keys = 32;   // keys per LDS block

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillParams p) {
  __shared__ float q_s[kF32Rows][D + 1];
  __shared__ float k_s[kF32Keys][D];
  __shared__ float v_s[kF32Keys][D];

  const int lane = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (p.Hq / p.Hkv);
  int n = p.Skv;
  if (p.kv_lens) n = min(max(p.kv_lens[b], 0), p.Skv);

  const float* qp = static_cast<const float*>(p.q) + ((int64_t)b * p.Hq + h) * p.Sq * D;
  const float* kp = static_cast<const float*>(p.k) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  const float* vp = static_cast<const float*>(p.v) + ((int64_t)b * p.Hkv + g) * p.Skv * D;
  float* op = static_cast<float*>(p.o) + ((int64_t)b * p.Hq + h) * p.Sq * D;

  const int row0 = qt * kF32Rows;
  for (int r = 0; r < kF32Rows; ++r) {
    const int row = row0 + r;
    for (int c = lane; c < D; c += 64) q_s[r][c] = row < p.Sq ? qp[(int64_t)row * D + c] : 0.f;
  }

  const int i = row0 + lane;                       // this lane's query row
  const int last_row = min(row0 + kF32Rows, p.Sq) - 1;
  int kend = n;                                    // keys any row of the tile may see
  if (CAUSAL) kend = min(n, max(0, last_row + n - p.Sq + 1));
  const int my_last = CAUSAL ? i + n - p.Sq : n - 1;  // last key this row sees

  float m = kNegInf, l = 0.f;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;

  for (int j0 = 0; j0 < kend; j0 += kF32Keys) {
    __syncthreads();
    for (int r = 0; r < kF32Keys; ++r) {
      const int64_t row = min(j0 + r, n - 1);       // clamp: masked rows read a valid row
      for (int c = lane; c < D; c += 64) {
        k_s[r][c] = kp[row * D + c];
        v_s[r][c] = vp[row * D + c];
      }
    }
    __syncthreads();

    float s[kF32Keys];
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) s[r] = 0.f;
    for (int c = 0; c < D; ++c) {
      const float qc = q_s[lane][c];
#pragma unroll
      for (int r = 0; r < kF32Keys; ++r) s[r] = fmaf(qc, k_s[r][c], s[r]);
    }
    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      const int j = j0 + r;
      const bool vis = j < n && j <= my_last;
      s[r] = vis ? s[r] * p.scale_log2 : kNegInf;
      mt = fmaxf(mt, s[r]);
    }
    const float m_new = fmaxf(m, mt);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2_fast(m - m_use);
    l *= alpha;
#pragma unroll
    for (int r = 0; r < kF32Keys; ++r) {
      s[r] = exp2_fast(s[r] - m_use);
      l += s[r];
    }
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float a = acc[c] * alpha;
#pragma unroll
      for (int r = 0; r < kF32Keys; ++r) a = fmaf(s[r], v_s[r][c], a);
      acc[c] = a;
    }
    m = m_new;
  }

  if (i < p.Sq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      f32x4 w = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
      *reinterpret_cast<f32x4*>(op + (int64_t)i * D + c) = w;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const PrefillParams& p, hipStream_t stream) {
  dim3 grid((p.Sq + kF32Rows - 1) / kF32Rows, p.Hq, p.B);
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream) {
  if (p.d == 64) return p.causal ? launch<64, true>(p, stream) : launch<64, false>(p, stream);
  return p.causal ? launch<128, true>(p, stream) : launch<128, false>(p, stream);
}

}  // namespace attn

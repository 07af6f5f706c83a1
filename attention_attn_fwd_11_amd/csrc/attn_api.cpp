// attn_api.cpp -- the C ABI (include/attn.h): argument validation, launch
// configuration and error reporting.  All checks run on the host before any
// HIP call, so an invalid call launches nothing and touches no memory.
#include "../../include/attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

namespace {

thread_local char g_hip_error[256] = "";

attn_status_t hip_fail(const char* what, hipError_t e) {
  std::snprintf(g_hip_error, sizeof g_hip_error, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
  return ATTN_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared size checks for both entry points.
attn_status_t check_common(const void* q, const void* k, const void* v, const void* o, int32_t B,
                           int32_t H_q, int32_t H_kv, int32_t S_q, int32_t S_kv, int32_t d,
                           int32_t causal, float scale, int dtype) {
  if (B < 0 || S_q < 0 || S_kv < 0 || H_q < 1 || H_kv < 1 || d < 1) return ATTN_ERR_SHAPE;
  if (H_q % H_kv != 0) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_VALUE;
  const bool has_q = (int64_t)B * S_q > 0;
  const bool has_kv = (int64_t)B * S_kv > 0;
  if (has_q && (!q || !o)) return ATTN_ERR_NULL;
  if (has_kv && (!k || !v)) return ATTN_ERR_NULL;
  if ((q && !aligned16(q)) || (o && !aligned16(o)) || (k && !aligned16(k)) || (v && !aligned16(v)))
    return ATTN_ERR_ALIGN;
  // Within one head the kernels use 32-bit byte offsets (buffer loads among
  // them), so each head's rows of q, k, v, o must span at most 2^31 - 1 bytes.
  const int64_t elem = dtype == ATTN_F32 ? 4 : 2;
  if ((int64_t)S_kv * d * elem > INT32_MAX || (int64_t)S_q * d * elem > INT32_MAX) return ATTN_ERR_SHAPE;
  if ((int64_t)B * H_q > INT32_MAX / 2) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

// The decode kernels and the fp32 prefill index batches and heads by the
// grid's second and third dimensions, which the device limits to 65536.
constexpr int32_t kMaxGridYZ = 65535;
bool grid_yz_ok(int32_t B, int32_t H_q) { return B <= kMaxGridYZ && H_q <= kMaxGridYZ; }

// Causal prefill: pair query tiles n_qt-1-p and p in one workgroup when the
// queries span at least half of the keys (the tiles' work then grows along
// the diagonal and the pairs even it out); a short chunk of queries at the
// end of a long cache has tiles of nearly equal work, where pairing would
// only halve the number of workgroups.
int pair_tiles(int32_t causal, int32_t S_q, int32_t S_kv) {
  return causal && 2LL * S_q >= S_kv ? 1 : 0;
}

// Query groups (G = H_q / H_kv >= 2) run on the matrix cores in column
// blocks of at most 16 query heads: *blocks per KV head and *cb query heads
// per block (the last block of a head may hold fewer).  One block of G for
// G <= 16.
void group_blocks(int32_t H_q, int32_t H_kv, int* blocks, int* cb) {
  const int G = H_q / H_kv;
  *blocks = (G + 15) / 16;
  *cb = (G + *blocks - 1) / *blocks;
}

// Virtual KV heads of the matrix-core pass (H_kv times the blocks per head).
int64_t virtual_heads(int32_t H_q, int32_t H_kv) {
  int blocks = 1, cb = 1;
  group_blocks(H_q, H_kv, &blocks, &cb);
  return (int64_t)H_kv * blocks;
}

// Query groups run on the matrix cores; one query head per KV head on the
// vector-ALU pass.
bool mfma_group(int32_t H_q, int32_t H_kv, int32_t d) {
  (void)d;
  return H_q / H_kv >= 2;
}

// Decode work decomposition.  Matrix-core query groups with at most
// kDecodeMaxBatch sequences use the balanced pass: fixed units of
// kDecodeUnit keys spread evenly over a persistent grid.  Otherwise the cache
// is split into equal chunks per (batch, head): KV head for the matrix-core
// kernels, query head for the vector-ALU one.
bool decode_balanced(int32_t B, int32_t H_q, int32_t H_kv, int32_t d) {
  return mfma_group(H_q, H_kv, d) && B <= attn::kDecodeMaxBatch;
}

// Keys per split (or per unit on the balanced pass).  Test-only override for
// the chunked pass: ATTN_DECODE_CHUNK (a positive multiple of 256) forces the
// chunk so split-count invariance can be tested.
int decode_chunk(int32_t B, int32_t H_q, int32_t H_kv, int32_t S_kv, int32_t d) {
  if (decode_balanced(B, H_q, H_kv, d)) return attn::kDecodeUnit;
  if (const char* env = std::getenv("ATTN_DECODE_CHUNK")) {
    const long c = std::strtol(env, nullptr, 10);
    if (c >= 256 && c % 256 == 0 && c <= (1 << 30)) return (int)c;
  }
  // Aim for about 4096 workgroups (16 per compute unit on a 256-CU part), so
  // the cache of every head is split even at B64 H32, but never split below
  // 512 keys: each split costs a partial (d+1 floats) per query.  (For B64
  // H32 L4096 one split per head would stream at 6.95 TB/s, two, as chosen,
  // at 6.86, four at 6.75.)
  const int64_t heads = (int64_t)B * (mfma_group(H_q, H_kv, d) ? virtual_heads(H_q, H_kv) : H_q);
  int64_t splits = heads >= 4096 ? 1 : (4096 + heads - 1) / heads;
  const int64_t max_splits = (S_kv + 511) / 512;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t chunk = (S_kv + splits - 1) / splits;
  chunk = (chunk + 255) / 256 * 256;
  if (chunk < 256) chunk = 256;
  return (int)chunk;
}

// Compute units of the current device, queried once per device.
int device_cus(int* dev_out) {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  *dev_out = dev;
  if (dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return -1;
    cus[dev] = n;
  }
  return cus[dev];
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Partial rows (one per split and query head, or per run and query head on
// the balanced pass) a decode of this shape may write.
size_t partial_rows(int32_t B, int32_t H_q, int32_t H_kv, int32_t S_kv, int32_t d) {
  const int chunk = decode_chunk(B, H_q, H_kv, S_kv, d);
  const int64_t n_split = (S_kv + chunk - 1) / chunk;
  if (decode_balanced(B, H_q, H_kv, d)) {
    // a run per (virtual head, workgroup range) boundary: fewer than
    // B*Hv + n_wg, with n_wg at most kDecodeMaxWg and at most the number of
    // units; cb partial rows per run
    int blocks = 1, cb = 1;
    group_blocks(H_q, H_kv, &blocks, &cb);
    const int64_t hv = (int64_t)H_kv * blocks;
    int64_t wg = (int64_t)B * hv * n_split;
    if (wg > attn::kDecodeMaxWg) wg = attn::kDecodeMaxWg;
    return (size_t)((int64_t)B * hv + wg) * cb;
  }
  return (size_t)B * H_q * n_split;
}

size_t workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t S_kv, int32_t d) {
  if (B <= 0 || S_kv <= 0 || H_q < 1 || H_kv < 1 || H_q % H_kv != 0 || (d != 64 && d != 128 && d != 256))
    return 0;
  const size_t rows = partial_rows(B, H_q, H_kv, S_kv, d);
  return round_up(rows * d * sizeof(float), 256) + round_up(rows * sizeof(float), 256);
}

// What the decode kernels implement: d 64, 128 or 256, bf16 or fp32, any
// group size.
bool decode_supported(int32_t H_q, int32_t H_kv, int32_t d, attn_dtype_t dtype) {
  (void)H_q;
  (void)H_kv;
  if (d != 64 && d != 128 && d != 256) return false;
  return dtype == ATTN_F32 || dtype == ATTN_BF16;
}

// Scratch of the allocation-free decode entry point (attn_decode_noalloc_fwd):
// one copy per GPU the library runs on, held until the process ends.  Host
// code never passes `scratch` itself (in host code its name stands for a host
// shadow, not a device address); it uses the address static_scratch() looked
// up with hipGetSymbolAddress for the device the work runs on.
constexpr size_t kScratchBytes = ATTN_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on the device of `stream` (the current device
// for the null stream), looked up once per device with that device current.
attn_status_t static_scratch(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int cur = 0, dev = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail("hipStreamGetDevice", e);
  }
  if (dev < 0 || dev >= 64) return hip_fail("device index out of range", hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail("hipSetDevice", e);
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess && r != hipSuccess) e = r;
    }
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (!ptr) return hip_fail("hipGetSymbolAddress(scratch)", hipErrorInvalidSymbol);
    addr[dev] = ptr;
  }
  *out = addr[dev];
  return ATTN_OK;
}

// Decode after the entry point's own checks (shared by the contiguous and the
// paged cache; block_table == nullptr selects the contiguous layout).
attn_status_t run_decode(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H_q,
                         int32_t H_kv, int32_t S_kv, int32_t d, float scale, const int32_t* kv_lens,
                         attn_dtype_t dtype, void* workspace, size_t ws_bytes, void* stream,
                         const int32_t* block_table, int32_t max_blocks, int32_t page_size,
                         int32_t num_pages) {
  if (!decode_supported(H_q, H_kv, d, dtype)) return ATTN_ERR_UNSUPPORTED;
  if (B == 0) return ATTN_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (S_kv == 0) {
    const size_t elt = dtype == ATTN_F32 ? 4 : 2;
    hipError_t e = attn::launch_zero_fill(o, (size_t)B * H_q * d * elt, s);
    return e == hipSuccess ? ATTN_OK : hip_fail("zero-fill launch", e);
  }
  const size_t need = workspace_bytes(B, H_q, H_kv, S_kv, d);
  if (!workspace || ws_bytes < need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  if (dtype == ATTN_F32) {
    // fp32: every query head streams its own chunks (the one-head-per-KV-head
    // split policy applied to the query heads), with no more splits than the
    // workspace that attn_decode_workspace_bytes sized holds (at least one
    // per query head for every group size).  Chunks are multiples of 256 keys.
    attn::DecodeParams p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.kv_lens = kv_lens;
    p.B = B; p.Hq = H_q; p.Hkv = H_kv; p.Skv = S_kv; p.d = d;
    p.block_table = block_table; p.max_blocks = max_blocks; p.page_size = page_size;
    p.num_pages = num_pages;
    const size_t rows = partial_rows(B, H_q, H_kv, S_kv, d);
    int64_t splits = (S_kv + decode_chunk(B, H_q, H_q, S_kv, d) - 1) / decode_chunk(B, H_q, H_q, S_kv, d);
    const int64_t fit = (int64_t)(rows / ((size_t)B * H_q));
    if (splits > fit) splits = fit;
    if (splits < 1) splits = 1;
    int64_t chunk = (S_kv + splits - 1) / splits;
    chunk = (chunk + 255) / 256 * 256;
    p.chunk = (int)chunk;
    p.n_split = (int)((S_kv + chunk - 1) / chunk);
    p.part_o = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                          round_up(rows * d * sizeof(float), 256));
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipError_t e = attn::launch_decode_f32(p, s);
    return e == hipSuccess ? ATTN_OK : hip_fail("decode launch", e);
  }

  attn::DecodeParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.kv_lens = kv_lens;
  p.B = B; p.Hq = H_q; p.Hkv = H_kv; p.Skv = S_kv; p.d = d;
  p.block_table = block_table; p.max_blocks = max_blocks; p.page_size = page_size;
  p.num_pages = num_pages;
  p.chunk = decode_chunk(B, H_q, H_kv, S_kv, d);
  p.n_split = (S_kv + p.chunk - 1) / p.chunk;
  p.n_wg = 0;
  group_blocks(H_q, H_kv, &p.kv_div, &p.cb);
  p.Hv = H_kv * p.kv_div;
  if (decode_balanced(B, H_q, H_kv, d)) {
    // Persistent grid: the resident capacity (two workgroups per compute
    // unit, one at d = 256), never more than there are units.  The contiguous and the paged cache use the same
    // grid, so both partition the keys alike and give the same bits.
    // Test-only override: ATTN_DECODE_WORKGROUPS.
    int dev = 0;
    const int cus = device_cus(&dev);
    if (cus <= 0) return hip_fail("hipDeviceGetAttribute(multiprocessor count)", hipGetLastError());
    int64_t wg = (int64_t)attn::decode_wg_per_cu(d) * cus;
    if (const char* env = std::getenv("ATTN_DECODE_WORKGROUPS")) {
      const long w = std::strtol(env, nullptr, 10);
      if (w >= 1 && w <= (1 << 20)) wg = w;
    }
    const int64_t max_units = (int64_t)B * p.Hv * p.n_split;
    if (wg > max_units) wg = max_units;
    if (wg > attn::kDecodeMaxWg) wg = attn::kDecodeMaxWg;
    p.n_wg = (int)wg;
  }
  const size_t rows = partial_rows(B, H_q, H_kv, S_kv, d);
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        round_up(rows * d * sizeof(float), 256));
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  hipError_t e = attn::launch_decode_bf16(p, s);
  return e == hipSuccess ? ATTN_OK : hip_fail("decode launch", e);
}

}  // namespace

extern "C" {

const char* attn_status_str(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "inconsistent or invalid sizes";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    case ATTN_ERR_VALUE: return "non-finite scale";
  }
  return "unknown status";
}

const char* attn_last_hip_error(void) { return g_hip_error; }

size_t attn_prefill_rope_workspace_bytes(int32_t B, int32_t H_kv, int32_t S_kv, int32_t d) {
  if (B < 0 || H_kv < 0 || S_kv < 0 || d < 0) return 0;
  return (size_t)B * H_kv * S_kv * d * 2;
}

size_t attn_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t S_kv, int32_t d) {
  return workspace_bytes(B, H_q, H_kv, S_kv, d);
}

attn_status_t attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, int32_t B,
                               int32_t H_q, int32_t H_kv, int32_t S_q, int32_t S_kv, int32_t d,
                               int32_t causal, float scale, const int32_t* kv_lens,
                               attn_dtype_t dtype, void* stream) {
  g_hip_error[0] = '\0';
  attn_status_t st = check_common(q, k, v, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (causal && S_q > S_kv) return ATTN_ERR_SHAPE;
  if (dtype == ATTN_F32 && !grid_yz_ok(B, H_q)) return ATTN_ERR_SHAPE;
  if ((int64_t)B * S_q == 0) return ATTN_OK;  // nothing to compute
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (S_kv == 0) {
    // every row sees no key: O = 0
    const size_t elt = dtype == ATTN_F32 ? 4 : 2;
    hipError_t e = attn::launch_zero_fill(o, (size_t)B * H_q * S_q * d * elt, s);
    return e == hipSuccess ? ATTN_OK : hip_fail("zero-fill launch", e);
  }
  attn::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.kv_lens = kv_lens;
  p.B = B; p.Hq = H_q; p.Hkv = H_kv; p.Sq = S_q; p.Skv = S_kv; p.d = d; p.causal = causal;
  p.pair = pair_tiles(causal, S_q, S_kv);
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  hipError_t e = dtype == ATTN_F32 ? attn::launch_prefill_f32(p, s) : attn::launch_prefill_bf16(p, s);
  return e == hipSuccess ? ATTN_OK : hip_fail("prefill launch", e);
}

attn_status_t attn_prefill_rope_fwd(const void* q, const void* k, const void* v, void* o, int32_t B,
                                    int32_t H_q, int32_t H_kv, int32_t S_q, int32_t S_kv, int32_t d,
                                    int32_t causal, float scale, const int32_t* kv_lens,
                                    const float* rope_table, int32_t rope_rows, void* workspace,
                                    size_t workspace_bytes, attn_dtype_t dtype, void* stream) {
  g_hip_error[0] = '\0';
  attn_status_t st = check_common(q, k, v, o, B, H_q, H_kv, S_q, S_kv, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (causal && S_q > S_kv) return ATTN_ERR_SHAPE;
  if (rope_rows < S_kv || rope_rows < 1) return ATTN_ERR_SHAPE;   // every key position has a row
  if ((int64_t)B * S_q > 0 && S_kv > 0 && !rope_table) return ATTN_ERR_NULL;
  if (rope_table && !aligned16(rope_table)) return ATTN_ERR_ALIGN;
  if (workspace) {
    if (workspace_bytes < attn_prefill_rope_workspace_bytes(B, H_kv, S_kv, d)) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  }
  if ((int64_t)B * S_q == 0) return ATTN_OK;  // nothing to compute
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (S_kv == 0) {
    hipError_t e = attn::launch_zero_fill(o, (size_t)B * H_q * S_q * d * 2, s);
    return e == hipSuccess ? ATTN_OK : hip_fail("zero-fill launch", e);
  }
  attn::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.kv_lens = kv_lens;
  p.B = B; p.Hq = H_q; p.Hkv = H_kv; p.Sq = S_q; p.Skv = S_kv; p.d = d; p.causal = causal;
  p.pair = pair_tiles(causal, S_q, S_kv);
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.rope = rope_table; p.rope_rows = rope_rows;
  p.rope_k = workspace ? 0 : 1;
  if (workspace) {   // keys rotated once into the workspace, Q in the kernel
    hipError_t e = attn::launch_rope_rows(k, workspace, rope_table, kv_lens, B, H_kv, S_kv, d, s);
    if (e != hipSuccess) return hip_fail("rope launch", e);
    p.k = workspace;
  }
  hipError_t e = attn::launch_prefill_bf16(p, s);
  return e == hipSuccess ? ATTN_OK : hip_fail("prefill launch", e);
}

attn_status_t attn_prefill_varlen_fwd(const void* q, const void* k, const void* v, void* o,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      int32_t B, int32_t H_q, int32_t H_kv, int32_t max_seqlen_q,
                                      int32_t max_seqlen_k, int32_t total_q, int32_t total_k,
                                      int32_t d, int32_t causal, float scale, attn_dtype_t dtype,
                                      void* stream) {
  g_hip_error[0] = '\0';
  if (B < 0 || H_q < 1 || H_kv < 1 || max_seqlen_q < 0 || max_seqlen_k < 0 || total_q < 0 ||
      total_k < 0)
    return ATTN_ERR_SHAPE;
  if (H_q % H_kv != 0) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_ERR_VALUE;
  const bool has_q = (int64_t)B * max_seqlen_q > 0 && total_q > 0;
  const bool has_kv = (int64_t)B * max_seqlen_k > 0 && total_k > 0;
  if (B > 0 && (!cu_seqlens_q || !cu_seqlens_k)) return ATTN_ERR_NULL;
  if (has_q && (!q || !o)) return ATTN_ERR_NULL;
  if (has_q && has_kv && (!k || !v)) return ATTN_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return ATTN_ERR_ALIGN;
  if ((q && !aligned16(q)) || (o && !aligned16(o)) || (k && !aligned16(k)) || (v && !aligned16(v)))
    return ATTN_ERR_ALIGN;
  // K/V rows of one sequence and head are addressed with 32-bit byte offsets.
  if ((int64_t)max_seqlen_k * H_kv * d * 2 > INT32_MAX) return ATTN_ERR_SHAPE;
  if ((int64_t)B * H_q > INT32_MAX / 2) return ATTN_ERR_SHAPE;
  if (!has_q) return ATTN_OK;  // nothing to compute
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!has_kv) {
    // no sequence has a key: every row of O is 0
    hipError_t e = attn::launch_zero_fill(o, (size_t)total_q * H_q * d * 2, s);
    return e == hipSuccess ? ATTN_OK : hip_fail("zero-fill launch", e);
  }
  attn::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.o = o; p.kv_lens = nullptr;
  p.B = B; p.Hq = H_q; p.Hkv = H_kv; p.Sq = max_seqlen_q; p.Skv = max_seqlen_k; p.d = d;
  p.causal = causal;
  // Pairs even out the tiles of one sequence, but over sequences of unequal
  // lengths single tiles, heaviest first, balance the grid better (16
  // sequences of U[256, 4096] tokens: 1.110 -> 0.987 ms).  Every sequence has
  // the maximum lengths exactly when the totals say so.
  const bool uniform = (int64_t)total_q == (int64_t)B * max_seqlen_q &&
                       (int64_t)total_k == (int64_t)B * max_seqlen_k;
  p.pair = uniform ? pair_tiles(causal, max_seqlen_q, max_seqlen_k) : 0;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);
  p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k; p.total_q = total_q; p.total_k = total_k;
  hipError_t e = attn::launch_prefill_bf16(p, s);
  return e == hipSuccess ? ATTN_OK : hip_fail("prefill launch", e);
}

attn_status_t attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, void* o,
                              int32_t B, int32_t H_q, int32_t H_kv, int32_t S_q, int32_t S_kv,
                              int32_t d, int32_t causal, float scale, const int32_t* kv_lens,
                              attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream) {
  g_hip_error[0] = '\0';
  attn_status_t st = check_common(q, k_cache, v_cache, o, B, H_q, H_kv, S_q, S_kv, d, causal,
                                  scale, dtype);
  if (st != ATTN_OK) return st;
  if (S_q != 1 || !grid_yz_ok(B, H_q)) return ATTN_ERR_SHAPE;
  return run_decode(q, k_cache, v_cache, o, B, H_q, H_kv, S_kv, d, scale, kv_lens, dtype, workspace,
                    workspace_bytes, stream, nullptr, 0, 0, 0);
}

attn_status_t attn_decode_noalloc_fwd(const void* q, const void* k_cache, const void* v_cache,
                                      void* o, int32_t B, int32_t H_q, int32_t H_kv, int32_t S_q,
                                      int32_t S_kv, int32_t d, int32_t causal, float scale,
                                      const int32_t* kv_lens, attn_dtype_t dtype, void* stream) {
  g_hip_error[0] = '\0';
  attn_status_t st = check_common(q, k_cache, v_cache, o, B, H_q, H_kv, S_q, S_kv, d, causal,
                                  scale, dtype);
  if (st != ATTN_OK) return st;
  if (S_q != 1 || !grid_yz_ok(B, H_q)) return ATTN_ERR_SHAPE;
  if (!decode_supported(H_q, H_kv, d, dtype)) return ATTN_ERR_UNSUPPORTED;
  const size_t need = workspace_bytes(B, H_q, H_kv, S_kv, d);
  if (need > kScratchBytes) return ATTN_ERR_WORKSPACE;   // beyond the static scratch
  void* ws = nullptr;
  if (need > 0) {
    st = static_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != ATTN_OK) return st;
  }
  return run_decode(q, k_cache, v_cache, o, B, H_q, H_kv, S_kv, d, scale, kv_lens, dtype, ws,
                    kScratchBytes, stream, nullptr, 0, 0, 0);
}

attn_status_t attn_decode_paged_fwd(const void* q, const void* k_pages, const void* v_pages, void* o,
                                    int32_t B, int32_t H_q, int32_t H_kv, int32_t d, float scale,
                                    const int32_t* block_table, int32_t max_blocks,
                                    int32_t page_size, int32_t num_pages, const int32_t* kv_lens,
                                    attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  g_hip_error[0] = '\0';
  if (page_size < attn::kDecodeUnit || page_size % attn::kDecodeUnit != 0 || max_blocks < 1 ||
      num_pages < 1)
    return ATTN_ERR_SHAPE;
  const int64_t cap = (int64_t)max_blocks * page_size;
  if (cap > INT32_MAX) return ATTN_ERR_SHAPE;
  attn_status_t st = check_common(q, k_pages, v_pages, o, B, H_q, H_kv, 1, (int32_t)cap, d, 0,
                                  scale, dtype);
  if (st != ATTN_OK) return st;
  if (!grid_yz_ok(B, H_q)) return ATTN_ERR_SHAPE;
  if (B > 0 && !block_table) return ATTN_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(block_table) & 3u) return ATTN_ERR_ALIGN;
  return run_decode(q, k_pages, v_pages, o, B, H_q, H_kv, (int32_t)cap, d, scale, kv_lens, dtype,
                    workspace, workspace_bytes, stream, block_table, max_blocks, page_size,
                    num_pages);
}

}  // extern "C"

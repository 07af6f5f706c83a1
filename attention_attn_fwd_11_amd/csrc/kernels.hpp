// kernels.hpp -- host-side launch interface between the C ABI layer and the
// kernels.  Every launcher assumes its arguments were validated by the ABI
// layer (sizes, alignment, supported d and dtype) and only enqueues work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* kv_lens;  // device int32[B] or nullptr
  int B, Hq, Hkv, Sq, Skv, d;
  int causal;
  float scale_log2;        // scale * log2(e)
  // Packed sequences (cu_q != nullptr, bf16 only): q, o are [total_q, Hq, d]
  // and k, v [total_k, Hkv, d]; sequence b owns rows [cu_q[b], cu_q[b+1]) and
  // [cu_k[b], cu_k[b+1]).  Sq and Skv are then the largest lengths.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  // Rotary embedding (rope != nullptr, bf16 only): table [rope_rows, d] fp32,
  // columns f < d/2 the cos and d/2 + f the sin of position p's angle for
  // frequency f; Q and K are rotated (rotate-half pairs) before the scores.
  // rope_k = 0: k already holds rotated keys (launch_rope_rows), so only Q
  // is rotated in the kernel.
  const float* rope;
  int rope_rows;
  int rope_k;
  // Causal only: 1 = one workgroup takes query tiles n_qt-1-p and p (equal
  // work per workgroup when queries and keys span the same positions); 0 =
  // one tile per workgroup, heaviest first (a chunk of queries at the end of
  // a long cache, where every tile has about the same work).
  int pair;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const int32_t* kv_lens;  // device int32[B] or nullptr
  // Chunked pass: [B, Hq, n_split, d] and [B, Hq, n_split]; balanced pass:
  // [B * Hv + n_wg, cb, d] and [B * Hv + n_wg, cb] (one slot per run).
  float* part_o;           // fp32 partial outputs, normalised
  float* part_lse;         // fp32 base-2 log-sum-exps
  int B, Hq, Hkv, Skv, d;
  int chunk;               // keys per split (G = 1) or per unit (G >= 2)
  int n_split;             // partial slots per (batch, query head)
  int n_wg;                // G >= 2: workgroups of the balanced split pass
  float scale_log2;
  // Paged cache (block_table != nullptr): k and v are page pools
  // [num_pages, Hkv, page_size, d]; row j of batch b lives in page
  // block_table[b * max_blocks + j / page_size] at row j % page_size.
  // page_size is a multiple of kDecodeUnit; Skv = max_blocks * page_size.
  const int32_t* block_table;
  int max_blocks, page_size, num_pages;
  // Query groups on the matrix cores (G = Hq / Hkv >= 2) are cut into
  // kv_div column blocks of at most 16 query heads: virtual KV head vh
  // (Hv = Hkv * kv_div of them) reads KV head vh / kv_div and holds query
  // heads (vh / kv_div) * G + (vh % kv_div) * cb .. of it, cb of them (the
  // last block of a head may hold fewer).  Groups of 2, 4, 8, 16: kv_div = 1,
  // cb = G, Hv = Hkv.
  int Hv, kv_div, cb;
};

// Largest batch the balanced (G >= 2) decode pass handles: its workgroups
// keep a prefix sum of per-batch work in LDS.
constexpr int kDecodeMaxBatch = 2048;
// Resident workgroups per compute unit the balanced decode pass is built for
// (its register bound) and launched with (its persistent grid): each stages
// a K and a V block per wave in LDS, 64 KiB per workgroup.
constexpr int kDecodeWgPerCu = 2;
// At d = 256 the staging doubles (128 KiB per workgroup): one per compute unit.
constexpr int decode_wg_per_cu(int d) { return d == 256 ? 1 : kDecodeWgPerCu; }
// Keys per work unit of the balanced decode pass (4 waves x 32 keys).
constexpr int kDecodeUnit = 128;
// Most workgroups of the balanced decode pass; its partials need at most
// B * H_kv + (workgroups) slots per query head of a group.
constexpr int kDecodeMaxWg = 1024;

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);
// d = 256 without the rotary embedding (16-row waves; called by launch_prefill_bf16)
hipError_t launch_prefill_d256(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);
// fp32 inputs and output (chunked split + combine, one workgroup per query head)
hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t stream);
hipError_t launch_zero_fill(void* dst, size_t bytes, hipStream_t stream);
// Rotary embedding of key rows into dst (same [B, H, S, d] bf16 layout as
// src): row j of every head at position j; rows j >= kv_lens[b] (when given)
// are skipped.
hipError_t launch_rope_rows(const void* src, void* dst, const float* table, const int32_t* kv_lens,
                            int B, int H, int S, int d, hipStream_t stream);

}  // namespace attn

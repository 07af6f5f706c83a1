/*
 * attn.h -- C ABI of the fused attention forward pass for MI355X (gfx950).
 *
 * The operation is exact softmax attention, O = softmax(Q K^T * scale + mask) V,
 * as defined in "GPU learning day 24: Operator Fusion" (daoyuly.cn), section
 * 3.4 (the standard attention block: scores, scaling and mask, softmax, P V),
 * and computed the way that section's FlashAttention loop does: K/V blocks
 * streamed through on-chip memory with a running row max and row sum, so the
 * score matrix is never written to device memory.  Decode follows "Optimizing
 * Decoder Attention for LLMs on GPU" (magmadev.ru), structure of attention in
 * decoding mode (one new query attends to all cached tokens), with the KV
 * sequence split into parallel parts as in the first page's FAQ Q4
 * (Flash-Decoding) and the parts merged by their log-sum-exp.
 *
 * Conventions shared by every entry point
 *   - Layout: contiguous row-major, head dimension innermost.
 *       Q, O : [B, H_q,  S_q,  d]
 *       K, V : [B, H_kv, S_kv, d]
 *     O has Q's dtype.  Accumulation is fp32 for every dtype.
 *   - Grouped-query attention: query head h reads KV head h / (H_q / H_kv).
 *   - Masking: the dot product is multiplied by `scale` first; masked keys
 *     then get weight exactly 0.  With kv_lens, batch b sees only its first
 *     n_b = clamp(kv_lens[b], 0, S_kv) keys.  `causal` aligns the mask to the
 *     bottom right: query i sees key j iff j <= i + n_b - S_q.  A row that sees
 *     no key is written as 0.
 *   - Pointers: device pointers, 16-byte aligned.  Buffers are owned by the
 *     caller; the library allocates nothing (attn_decode_noalloc_fwd uses a
 *     static array of its own), keeps no pointer after a call returns, and only enqueues work on `stream` (a hipStream_t; NULL means
 *     the null stream).  The caller keeps buffers alive until the stream has
 *     run the work.  A pointer may be NULL only when its tensor has no
 *     elements.
 *   - kv_lens: device int32[B] or NULL (NULL: every batch has S_kv keys).
 *     Its values are read on the device and clamped to [0, S_kv]; the host
 *     cannot check them without synchronising, so this is a precondition.
 *   - Errors: every function returns a status and never aborts or throws.
 *     All validation runs on the host before anything is launched; on any
 *     error nothing is launched and O is untouched.  ATTN_ERR_HIP means a HIP
 *     call failed; attn_last_hip_error() then names it.
 *   - Thread safety: the library is stateless apart from a per-device cache
 *     of the compute-unit count (filled once), a thread-local error string
 *     and the static scratch of attn_decode_noalloc_fwd (see there).
 *     Concurrent calls on different streams are safe, except that
 *     allocation-free decodes on one GPU share its scratch.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                      */
    ATTN_ERR_SHAPE = 2,       /* inconsistent or negative sizes                  */
    ATTN_ERR_UNSUPPORTED = 3, /* valid but not implemented: d, dtype             */
    ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
    ATTN_ERR_WORKSPACE = 5,   /* a workspace missing or too small                */
    ATTN_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed      */
    ATTN_ERR_VALUE = 7        /* non-finite scale                                */
} attn_status_t;

typedef enum {
    ATTN_F32 = 0,   /* IEEE binary32 in and out                             */
    ATTN_BF16 = 1   /* bfloat16 in and out (round to nearest even on output) */
} attn_dtype_t;

/*
 * Prefill (and general) attention forward.
 *
 *   q [B,H_q,S_q,d], k/v [B,H_kv,S_kv,d], o [B,H_q,S_q,d]   (device, dtype)
 *   B >= 0, S_q >= 0, S_kv >= 0, H_q >= 1, H_kv >= 1, H_q % H_kv == 0.
 *   One head's rows (S_q*d or S_kv*d elements) span at most 2^31 - 1 bytes,
 *   B*H_q <= 2^30 - 1, and with ATTN_F32 B <= 65535 and H_q <= 65535 (the
 *   grid dimensions the kernel indexes them by); else ATTN_ERR_SHAPE.
 *   d: 64, 128 or 256 (else ATTN_ERR_UNSUPPORTED).
 *   causal: 0 or 1; causal with S_q > S_kv is rejected (ATTN_ERR_SHAPE).
 *   scale: finite; the usual value is 1/sqrt(d).
 *   kv_lens: see above.
 *   dtype: ATTN_F32 or ATTN_BF16.  bf16 runs QK^T and PV on bf16 matrix cores
 *   with fp32 accumulation and rounds P to bf16 before PV; fp32 computes in
 *   fp32 throughout.
 *
 * Defined by the standard-attention block of "GPU learning day 24: Operator
 * Fusion", section 3.4, and computed by that section's tiled online-softmax
 * loop.
 */
attn_status_t attn_prefill_fwd(const void* q, const void* k, const void* v, void* o,
                               int32_t B, int32_t H_q, int32_t H_kv, int32_t S_q, int32_t S_kv,
                               int32_t d, int32_t causal, float scale, const int32_t* kv_lens,
                               attn_dtype_t dtype, void* stream);

/*
 * Attention forward with the rotary position embedding fused in (bf16).
 *
 *   Arguments as attn_prefill_fwd (dtype ATTN_BF16 only, else
 *   ATTN_ERR_UNSUPPORTED), plus
 *   rope_table: device fp32 [rope_rows, d], 16-byte aligned; row p holds
 *   cos(p * theta_f) in column f and sin(p * theta_f) in column d/2 + f for
 *   f < d/2.  rope_rows >= S_kv (else ATTN_ERR_SHAPE).
 * Each query and key row x at position p becomes
 *   (x[f] cos - x[f + d/2] sin, x[f + d/2] cos + x[f] sin),  f < d/2,
 * in fp32, rounded to bf16, before the scores.  Key j is at position j;
 * query i of a sequence with n keys at n - S_q + i (the causal mask's
 * bottom-right alignment; rows that see no key use position 0).  V is not
 * rotated.  "GPU learning day 24: Operator Fusion", section 6 (exercise 1's
 * reference answer), puts RoPE either in the QKV projection's epilogue or
 * inside the attention kernel; it gives no formula, and this is the
 * rotate-half form.  Q is always rotated inside the kernel, as its rows
 * are loaded.  K:
 *   workspace == NULL: each K stage is rotated in LDS inside the kernel
 *     (no extra memory; the work repeats for every query tile).
 *   workspace != NULL: device buffer of at least
 *     attn_prefill_rope_workspace_bytes(B, H_kv, S_kv, d) bytes (else
 *     ATTN_ERR_WORKSPACE), 16-byte aligned (else ATTN_ERR_ALIGN), owned by
 *     the caller and not read before the call: a first kernel writes the
 *     rotated keys there once (in place of the projection's epilogue) and
 *     the attention kernel reads them.  Rows past kv_lens[b] are left as
 *     they were.
 * Both give bit-identical O (the rotation is the same fp32 arithmetic).
 */
attn_status_t attn_prefill_rope_fwd(const void* q, const void* k, const void* v, void* o, int32_t B,
                                    int32_t H_q, int32_t H_kv, int32_t S_q, int32_t S_kv, int32_t d,
                                    int32_t causal, float scale, const int32_t* kv_lens,
                                    const float* rope_table, int32_t rope_rows, void* workspace,
                                    size_t workspace_bytes, attn_dtype_t dtype, void* stream);

/* Bytes of the key workspace attn_prefill_rope_fwd takes: B*H_kv*S_kv*d*2
 * (0 for a negative argument). */
size_t attn_prefill_rope_workspace_bytes(int32_t B, int32_t H_kv, int32_t S_kv, int32_t d);

/*
 * Attention forward over packed variable-length sequences (bf16).
 *
 *   q [total_q, H_q, d], o [total_q, H_q, d]; k, v [total_k, H_kv, d]
 *   (device, bf16, row-major: the H heads of a token are adjacent).
 *   cu_seqlens_q, cu_seqlens_k: device int32 [B+1], non-decreasing, starting
 *   at 0: sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and
 *   key rows [cu_seqlens_k[b], cu_seqlens_k[b+1]).  Their values are read on
 *   the device: offsets are clamped to [0, total], and a sequence's lengths
 *   to max_seqlen_q / max_seqlen_k, which must bound them.
 *   causal: bottom-right per sequence (query i of a sequence with s queries
 *   and n keys sees key j iff j <= i + n - s); a row that sees no key, also
 *   every row of a sequence with n = 0, gets O = 0.
 *   d: 64, 128 or 256; dtype: ATTN_BF16 only (else ATTN_ERR_UNSUPPORTED).
 *   max_seqlen_k * H_kv * d * 2 <= 2^31 - 1 (else ATTN_ERR_SHAPE).
 *   cu_seqlens_* must be 4-byte aligned, the tensors 16-byte aligned.
 *
 * Per sequence this is the operation of attn_prefill_fwd (the standard
 * attention of "GPU learning day 24: Operator Fusion", section 3.4), with the
 * same GQA head map; it runs the same kernel, with the row stride H*d and
 * each sequence's offsets in place of the padded [B, H, S, d] layout.
 */
attn_status_t attn_prefill_varlen_fwd(const void* q, const void* k, const void* v, void* o,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                      int32_t B, int32_t H_q, int32_t H_kv, int32_t max_seqlen_q,
                                      int32_t max_seqlen_k, int32_t total_q, int32_t total_k,
                                      int32_t d, int32_t causal, float scale, attn_dtype_t dtype,
                                      void* stream);

/*
 * Single-query decode over a KV cache.
 *
 *   q [B,H_q,1,d], o [B,H_q,1,d]; k_cache/v_cache [B,H_kv,S_kv,d] where S_kv is
 *   the cache capacity (the row stride between heads); batch b attends to its
 *   first clamp(kv_lens[b], 0, S_kv) rows.
 *   S_q must be 1, and B <= 65535 and H_q <= 65535 (the grid dimensions the
 *   kernels index them by); else ATTN_ERR_SHAPE.  causal is accepted and
 *   has no effect with one query row (the bottom-right mask then allows
 *   every key).  Size limits otherwise as attn_prefill_fwd.
 *   d: 64, 128 or 256 (else ATTN_ERR_UNSUPPORTED).  dtype: ATTN_BF16 or
 *   ATTN_F32, any group size H_q/H_kv; q, the caches and o all have that
 *   dtype.  bf16 computes scores and P V with fp32 accumulation; one query
 *   head per KV head on the vector ALU, larger groups on the matrix cores
 *   (P rounded to bf16 before P V) in blocks of at most 16 query heads, each
 *   block reading its KV head's rows once.  fp32 computes in fp32
 *   throughout.
 *   workspace: device memory of at least
 *   attn_decode_workspace_bytes(B, H_q, H_kv, S_kv, d) bytes, 16-byte
 *   aligned, for the per-split partial results (fp32).  Its contents need no
 *   initialisation and are scratch after the call.  Two calls that share a
 *   workspace must be ordered on one stream.
 *
 * Two kernels on `stream`: a split pass in which each workgroup streams one
 * chunk of the cache once and writes a normalised partial output with its
 * log-sum-exp, then a combine pass that merges the partials of each head
 * (the one-head-per-KV-head and fp32 passes skip it when every head has a
 * single split).
 * This is the Flash-Decoding split of "GPU learning day 24: Operator Fusion",
 * FAQ Q4, merged with the rescaling identity of that page's section 3.4 loop.
 */
attn_status_t attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, void* o,
                              int32_t B, int32_t H_q, int32_t H_kv, int32_t S_q, int32_t S_kv,
                              int32_t d, int32_t causal, float scale, const int32_t* kv_lens,
                              attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * Workspace bytes attn_decode_fwd needs for these sizes (0 if the sizes are
 * invalid or the problem is empty).  Pure host function; no HIP call.
 */
size_t attn_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t S_kv, int32_t d);

/*
 * Allocation-free single-query decode, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Arguments and results exactly as attn_decode_fwd, without the workspace:
 * the split partials go to a static device array of
 * ATTN_DECODE_NOALLOC_SCRATCH_BYTES bytes inside the library (one per GPU,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends).  A call whose attn_decode_workspace_bytes(B, H_q, H_kv, S_kv,
 * d) exceeds that size returns ATTN_ERR_WORKSPACE and launches nothing.  The
 * call allocates nothing (no hipMalloc, no hipFree); the first call on a GPU
 * looks up the array's device address once (hipGetSymbolAddress).  The
 * kernels are attn_decode_fwd's, so O is bitwise the same.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero).  Two calls that overlap
 * on one GPU -- on different streams, or on one stream inside graphs that
 * run concurrently -- race on it: order them on one stream.  The stream must
 * belong to a device whose copy of the library's code is loaded (any device
 * the process can use).
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
attn_status_t attn_decode_noalloc_fwd(const void* q, const void* k_cache, const void* v_cache,
                                      void* o, int32_t B, int32_t H_q, int32_t H_kv, int32_t S_q,
                                      int32_t S_kv, int32_t d, int32_t causal, float scale,
                                      const int32_t* kv_lens, attn_dtype_t dtype, void* stream);

/*
 * Single-query decode over a paged KV cache.
 *
 *   q [B,H_q,1,d], o [B,H_q,1,d]   (device, dtype)
 *   k_pages, v_pages: page pools [num_pages, H_kv, page_size, d] (device,
 *   dtype); page p holds page_size consecutive key rows of every KV head.
 *   block_table: device int32 [B, max_blocks]; key row j of sequence b is row
 *   j % page_size of page block_table[b * max_blocks + j / page_size].
 *   kv_lens: device int32[B] or NULL (NULL: every sequence has
 *   max_blocks * page_size keys); values are clamped to
 *   [0, max_blocks * page_size].  Only the table entries of pages that hold
 *   rows below a sequence's length are read; an entry outside
 *   [0, num_pages) is clamped into it (the result is then unspecified, but no
 *   memory outside the pools is read).
 *   page_size: a positive multiple of 128; max_blocks >= 1; num_pages >= 1
 *   (else ATTN_ERR_SHAPE).  max_blocks * page_size plays the role of S_kv in
 *   every other rule of attn_decode_fwd: the size limits, the dtypes and
 *   group sizes, d 64, 128 or 256, and the workspace, which
 *   must hold attn_decode_workspace_bytes(B, H_q, H_kv,
 *   max_blocks * page_size, d) bytes.  block_table must be 4-byte aligned
 *   (ATTN_ERR_ALIGN) and non-NULL when B > 0 (ATTN_ERR_NULL).
 *
 * The same split and combine kernels as attn_decode_fwd; only the address of
 * a key row changes (one table lookup per step of at most 64 keys, which
 * never straddles a page).  Results are bitwise identical to attn_decode_fwd
 * on the same keys laid out contiguously.  This is the decode step of
 * "Optimizing Decoder Attention for LLMs on GPU" (magmadev.ru) over a paged
 * KV cache, the PagedAttention layout that "What is kernel fusion and how is
 * it used in LLM serving?" (aivaro.ru), section 6 (tools and libraries),
 * lists for vLLM.  The pages give no layout; the pool order above keeps each
 * head's rows of a page contiguous.
 */
attn_status_t attn_decode_paged_fwd(const void* q, const void* k_pages, const void* v_pages, void* o,
                                    int32_t B, int32_t H_q, int32_t H_kv, int32_t d, float scale,
                                    const int32_t* block_table, int32_t max_blocks,
                                    int32_t page_size, int32_t num_pages, const int32_t* kv_lens,
                                    attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Static, NUL-terminated description of a status code. */
const char* attn_status_str(attn_status_t s);

/*
 * Text of the last HIP error seen by an attn_* call on this thread (the
 * failing call and hipGetErrorString), or "" if none.  Valid until the next
 * attn_* call on the same thread.
 */
const char* attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */

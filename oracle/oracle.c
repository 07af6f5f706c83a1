/*
 * oracle.c -- reference attention forward, for TESTING ONLY.
 *
 * This file is test infrastructure: only the test suite, the smoke check and
 * the CPU-baseline leg of the benchmark load it.  The product library never
 * links, loads or calls it, and it shares no code, header or constant with the
 * GPU kernels.
 *
 * What it computes is the plain definition of attention written out, in fp64:
 *
 *   "GPU learning day 24: Operator Fusion" (daoyuly.cn), section 3.4, the
 *   standard-attention block: S = Q K^T, then S / sqrt(d) + mask, then
 *   P = softmax(S), then O = P V.
 *
 *   "Optimizing Decoder Attention for LLMs on GPU" (magmadev.ru), section
 *   "Bottlenecks of traditional approaches", item 3: the softmax is taken in
 *   two passes, a max reduction and then the exponentiation and scaling.
 *
 * For every (b, h_q, i) row it runs three passes over a materialised score
 * row: (1) scores, (2) max, then exp and sum, then normalise, (3) P V.
 *
 * Readings where the pages are silent:
 *   - the dot product is multiplied by `scale` first, then the mask is added;
 *   - the mask is additive -inf, so a masked key gets weight exactly 0;
 *   - causal alignment is bottom-right: with len valid keys and S_q queries,
 *     query i may see key j iff j <= i + len - S_q;
 *   - grouped-query attention maps query head h to KV head h / (H_q / H_kv);
 *   - kv_lens[b] (if given) limits batch b to its first kv_lens[b] keys,
 *     clamped to [0, S_kv]; NULL means S_kv for every batch;
 *   - a row with no visible key has O = 0 and log-sum-exp -inf.
 *
 * Inputs are read in their stored format (fp64, fp32, or bf16 bit patterns)
 * and upcast exactly to fp64.  Outputs are fp64 and are not rounded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F64 = 0, ORACLE_F32 = 1, ORACLE_BF16 = 2 };

/* Exact upcast of element idx of a tensor stored in format dt. */
static double elem(const void* base, int dt, int64_t idx)
{
    if (dt == ORACLE_F64) return ((const double*)base)[idx];
    if (dt == ORACLE_F32) return (double)((const float*)base)[idx];
    /* bf16: the upper 16 bits of an IEEE binary32 */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *q, *k, *v;
    int dt;
    int B, Hq, Hkv, Sq, Skv, d, causal;
    double scale;
    const int32_t* kv_lens;
} problem_t;

/* Number of keys visible to query row i of batch b (keys 0 .. n-1). */
static int64_t visible_keys(const problem_t* P, int b, int i)
{
    int64_t len = P->Skv;
    if (P->kv_lens) {
        len = P->kv_lens[b];
        if (len < 0) len = 0;
        if (len > P->Skv) len = P->Skv;
    }
    int64_t n = len;
    if (P->causal) {
        int64_t last = (int64_t)i + len - P->Sq; /* last visible key index */
        if (last + 1 < n) n = last + 1;
        if (n < 0) n = 0;
    }
    return n;
}

/*
 * One output row: o[0..d) and its log-sum-exp.  s is caller scratch of at
 * least S_kv doubles.  If p_row is non-NULL it receives the S_kv
 * probabilities of the row (0 for masked keys).
 */
static void attend_row(const problem_t* P, int b, int h, int i,
                       double* s, double* o, double* lse, double* p_row)
{
    const int d = P->d;
    const int g = h / (P->Hq / P->Hkv);
    const int64_t qoff = (((int64_t)b * P->Hq + h) * P->Sq + i) * d;
    const int64_t kvbase = ((int64_t)b * P->Hkv + g) * (int64_t)P->Skv;
    const int64_t n = visible_keys(P, b, i);

    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (p_row)
        for (int64_t j = 0; j < P->Skv; ++j) p_row[j] = 0.0;
    if (n == 0) {
        *lse = -INFINITY;
        return;
    }

    /* pass 1: scores s_j = scale * <q_i, k_j> for the visible keys */
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        const int64_t koff = (kvbase + j) * d;
        for (int c = 0; c < d; ++c)
            acc += elem(P->q, P->dt, qoff + c) * elem(P->k, P->dt, koff + c);
        s[j] = P->scale * acc;
    }

    /* pass 2: max reduction, then exponentiate, sum and normalise */
    double m = s[0];
    for (int64_t j = 1; j < n; ++j)
        if (s[j] > m) m = s[j];
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t j = 0; j < n; ++j) s[j] /= l;
    *lse = m + log(l);
    if (p_row)
        for (int64_t j = 0; j < n; ++j) p_row[j] = s[j];

    /* pass 3: o = sum_j p_j v_j */
    for (int64_t j = 0; j < n; ++j) {
        const int64_t voff = (kvbase + j) * d;
        const double p = s[j];
        for (int c = 0; c < d; ++c) o[c] += p * elem(P->v, P->dt, voff + c);
    }
}

static int check(const problem_t* P)
{
    if (!P->q || !P->k || !P->v) return 1;
    if (P->dt < ORACLE_F64 || P->dt > ORACLE_BF16) return 2;
    if (P->B < 0 || P->Hq < 1 || P->Hkv < 1 || P->Sq < 0 || P->Skv < 0 || P->d < 1) return 3;
    if (P->Hq % P->Hkv != 0) return 4;
    return 0;
}

/*
 * Full attention.  Q, O: [B, H_q, S_q, d]; K, V: [B, H_kv, S_kv, d], all
 * contiguous row-major.  o: fp64 [B, H_q, S_q, d].  lse (optional): fp64
 * [B, H_q, S_q].  p (optional, tiny shapes): fp64 [B, H_q, S_q, S_kv].
 * Returns 0 on success, a positive code for invalid arguments.
 */
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     int B, int Hq, int Hkv, int Sq, int Skv, int d,
                     int causal, double scale, const int32_t* kv_lens,
                     double* o, double* lse, double* p)
{
    problem_t P = {q, k, v, dtype, B, Hq, Hkv, Sq, Skv, d, causal, scale, kv_lens};
    int rc = check(&P);
    if (rc) return rc;
    if (!o) return 1;
    const int64_t rows = (int64_t)B * Hq * Sq;
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t r = 0; r < rows; ++r) {
            if (!s) continue;
            const int i = (int)(r % Sq);
            const int h = (int)((r / Sq) % Hq);
            const int b = (int)(r / ((int64_t)Sq * Hq));
            double lse_r;
            attend_row(&P, b, h, i, s, o + r * d, &lse_r, p ? p + r * (int64_t)Skv : NULL);
            if (lse) lse[r] = lse_r;
        }
        free(s);
    }
    return bad ? 5 : 0;
}

/*
 * Selected rows only: sel holds n_rows (b, h_q, i) triples.  o_rows: fp64
 * [n_rows, d]; lse_rows (optional): fp64 [n_rows].  Used to check outputs of
 * shapes too large to evaluate in full.
 */
int oracle_attention_rows(const void* q, const void* k, const void* v, int dtype,
                          int B, int Hq, int Hkv, int Sq, int Skv, int d,
                          int causal, double scale, const int32_t* kv_lens,
                          const int64_t* sel, int64_t n_rows,
                          double* o_rows, double* lse_rows)
{
    problem_t P = {q, k, v, dtype, B, Hq, Hkv, Sq, Skv, d, causal, scale, kv_lens};
    int rc = check(&P);
    if (rc) return rc;
    if (!sel || !o_rows) return 1;
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t b = sel[3 * r], h = sel[3 * r + 1], i = sel[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Sq) return 6;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s) continue;
            double lse_r;
            attend_row(&P, (int)sel[3 * r], (int)sel[3 * r + 1], (int)sel[3 * r + 2],
                       s, o_rows + r * d, &lse_r, NULL);
            if (lse_rows) lse_rows[r] = lse_r;
        }
        free(s);
    }
    return bad ? 5 : 0;
}

/* Number of OpenMP threads the oracle will use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

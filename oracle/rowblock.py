"""Attention by its definition, one block of query rows at a time, with
library matrix products -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product library neither imports nor links it, and
the two share no code.

It computes exactly what oracle.c computes -- the standard attention of "GPU
learning day 24: Operator Fusion", section 3.4 (S = Q K^T, then S * scale plus
an additive mask, then P = softmax(S) row by row, then O = P V), with the
softmax taken in two passes as in "Optimizing Decoder Attention for LLMs on
GPU", section "Bottlenecks of traditional approaches", item 3 (a max
reduction, then exponentiation and normalisation) -- but the two products are
fp64 CPU matrix products (torch.matmul) over a block of query rows instead
of scalar loops, so that whole outputs of large problems can be evaluated.
The score block of `ROWS` query rows is materialised in full; every per-row
value is the one the scalar definition gives, up to the summation order the
library picks inside each dot product.

Readings where the pages are silent are the same as oracle.c's: scale first,
then the mask; the mask is additive -inf (a masked key has weight exactly 0);
causal alignment is bottom-right (with n valid keys and S_q queries, query i
sees key j iff j <= i + n - S_q); query head h reads KV head h / (H_q / H_kv);
kv_lens[b] limits batch b to its first kv_lens[b] keys (clamped to
[0, S_kv]); a row with no visible key is O = 0 with log-sum-exp -inf.

Inputs are CPU or device torch tensors (float64, float32, bfloat16) or numpy
arrays (float64, float32, uint16 holding bf16 bit patterns); they are
upcast exactly to float64 on the CPU.  Outputs are float64 numpy arrays.
"""
import numpy as np
import torch

IS_ROWBLOCK = True   # marks this module as an oracle implementation for oracle.attention(lib=...)
ROWS = 256           # query rows per materialised score block


def _f64(x):
    """Exact fp64 CPU copy of a stored tensor."""
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu()
        if x.dtype not in (torch.float64, torch.float32, torch.bfloat16):
            raise TypeError(f"unsupported tensor dtype {x.dtype}")
        return x.to(torch.float64).contiguous(), x.dtype
    a = np.ascontiguousarray(x)
    if a.dtype == np.uint16:   # bf16 bit patterns: the upper half of a binary32
        f = (a.astype(np.uint32) << 16).view(np.float32)
        return torch.from_numpy(f.astype(np.float64)), torch.bfloat16
    if a.dtype == np.float32:
        return torch.from_numpy(a.astype(np.float64)), torch.float32
    if a.dtype == np.float64:
        return torch.from_numpy(a.copy()), torch.float64
    raise TypeError(f"unsupported array dtype {a.dtype}")


def _inputs(q, k, v):
    (Q, tq), (K, tk), (V, tv) = _f64(q), _f64(k), _f64(v)
    if not (tq == tk == tv):
        raise TypeError("q, k, v must share one dtype")
    if Q.dim() != 4 or K.dim() != 4 or V.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, d]")
    B, Hq, _, d = Q.shape
    if K.shape != V.shape or K.shape[0] != B or K.shape[3] != d:
        raise ValueError("inconsistent q/k/v shapes")
    if K.shape[1] < 1 or Hq % K.shape[1] != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    return Q, K, V


def _lens(kv_lens, B, Skv):
    if kv_lens is None:
        return [Skv] * B
    if isinstance(kv_lens, torch.Tensor):
        kv_lens = kv_lens.detach().cpu().tolist()
    lens = [int(x) for x in np.asarray(kv_lens).reshape(-1)]
    if len(lens) != B:
        raise ValueError("kv_lens must have shape [B]")
    return [min(max(n, 0), Skv) for n in lens]


def _block(Qb, K, V, scale, first_row, n, Sq, causal, p_out=None):
    """Rows first_row .. first_row + len(Qb) - 1 of one (batch, head).

    K, V hold the n valid keys.  Returns (o [r, d], lse [r]); if p_out
    ([r, S_kv] float64) is given, the probabilities are written into it."""
    r, d = Qb.shape
    i = torch.arange(first_row, first_row + r, dtype=torch.int64)
    # number of keys each row sees: keys 0 .. last with last = i + n - S_q
    cnt = (i + (n - Sq) + 1).clamp(0, n) if causal else torch.full((r,), n, dtype=torch.int64)
    o = torch.zeros((r, d), dtype=torch.float64)
    lse = torch.full((r,), float("-inf"), dtype=torch.float64)
    kmax = int(cnt.max()) if r else 0
    if kmax == 0:
        return o, lse
    kmin = int(cnt.min())
    # pass 1: scores s_ij = scale * <q_i, k_j>, then the additive mask
    S = torch.matmul(Qb, K[:kmax].T)
    S.mul_(scale)
    if kmin < kmax:   # only the columns some row may not see
        j = torch.arange(kmin, kmax, dtype=torch.int64)
        S[:, kmin:].masked_fill_(j[None, :] >= cnt[:, None], float("-inf"))
    # pass 2: max per row, then exp(s - m), the row sum, and normalisation
    live = cnt > 0
    m = S.amax(dim=1)
    m = torch.where(live, m, torch.zeros_like(m))   # rows with no key: any finite shift
    S.sub_(m[:, None])
    S.exp_()
    l = S.sum(dim=1)
    S.div_(torch.where(live, l, torch.ones_like(l))[:, None])
    # pass 3: o_i = sum_j p_ij v_j
    o = torch.matmul(S, V[:kmax])
    o[~live] = 0.0
    lse = torch.where(live, m + torch.log(l), torch.full_like(m, float("-inf")))
    if p_out is not None:
        p_out[:, :kmax] = S
    return o, lse


def attention(q, k, v, causal, scale, kv_lens=None, want_lse=False, want_p=False):
    """Full fp64 attention.  Returns o [B,H_q,S_q,d] (and lse, p if asked)."""
    Q, K, V = _inputs(q, k, v)
    B, Hq, Sq, d = Q.shape
    Hkv, Skv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    lens = _lens(kv_lens, B, Skv)
    o = torch.zeros((B, Hq, Sq, d), dtype=torch.float64)
    lse = torch.full((B, Hq, Sq), float("-inf"), dtype=torch.float64)
    p = torch.zeros((B, Hq, Sq, Skv), dtype=torch.float64) if want_p else None
    for b in range(B):
        n = lens[b]
        for h in range(Hq):
            g = h // G
            Kb, Vb = K[b, g, :n], V[b, g, :n]
            for r0 in range(0, Sq, ROWS):
                r1 = min(Sq, r0 + ROWS)
                ob, lb = _block(Q[b, h, r0:r1], Kb, Vb, float(scale), r0, n, Sq, bool(causal),
                                None if p is None else p[b, h, r0:r1])
                o[b, h, r0:r1] = ob
                lse[b, h, r0:r1] = lb
    out = [o.numpy()]
    if want_lse:
        out.append(lse.numpy())
    if want_p:
        out.append(p.numpy())
    return out[0] if len(out) == 1 else tuple(out)


def attention_rows(q, k, v, causal, scale, rows, kv_lens=None, want_lse=False):
    """fp64 attention for selected (b, h_q, i) rows.  Returns o [n, d] (and lse [n])."""
    Q, K, V = _inputs(q, k, v)
    B, Hq, Sq, d = Q.shape
    Hkv, Skv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    lens = _lens(kv_lens, B, Skv)
    sel = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    bad = (sel < 0).any(axis=1) | (sel[:, 0] >= B) | (sel[:, 1] >= Hq) | (sel[:, 2] >= Sq)
    if bad.any():
        raise ValueError("selected row out of range")
    o = np.empty((sel.shape[0], d), np.float64)
    lse = np.empty((sel.shape[0],), np.float64)
    done = {}   # each row is taken from its whole ROWS-row block, as attention() forms it
    for r, (b, h, i) in enumerate(sel.tolist()):
        r0 = (i // ROWS) * ROWS
        key = (b, h, r0)
        if key not in done:
            n = lens[b]
            g = h // G
            done[key] = _block(Q[b, h, r0:min(Sq, r0 + ROWS)], K[b, g, :n], V[b, g, :n],
                               float(scale), r0, n, Sq, bool(causal))
        ob, lb = done[key]
        o[r] = ob[i - r0].numpy()
        lse[r] = float(lb[i - r0])
    return (o, lse) if want_lse else o


def decode(q, k_cache, v_cache, kv_lens, scale, want_lse=False):
    """Single-query decode: q [B,H_q,1,d] over the first kv_lens[b] cache rows."""
    if q.shape[2] != 1:
        raise ValueError("decode takes one query row per head")
    return attention(q, k_cache, v_cache, False, scale, kv_lens=kv_lens, want_lse=want_lse)

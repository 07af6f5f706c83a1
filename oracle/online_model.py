"""fp64 models of the tiled algorithms -- TEST INFRASTRUCTURE ONLY.

These are not the oracle (oracle.c is: the plain three-pass definition).
They restate, in numpy fp64, the algorithms the GPU kernels follow, so the
tests can check the pages' claim that the streaming form reaches the same
result as the standard form up to rounding ("GPU learning day 24: Operator
Fusion", FAQ Q1) before any kernel relies on it.

online_attention(): the tiled loop of section 3.4 of that page (FlashAttention:
tiling plus online softmax).  For each block of query rows, walk the key/value
blocks keeping a running row max m, a running row sum l and an unnormalised
accumulator; each block raises m to the block's max, rescales l and the
accumulator by exp(m_old - m_new), and adds the block's exponentials and their
product with V.  One division by l at the end.  Start values m = -inf, l = 0,
acc = 0; where m is still -inf the rescale factor is taken as 1 and masked
scores contribute 0.

split_combine_attention(): the split-KV decode of that page's FAQ Q4 (the
KV sequence dimension made parallel): every split of the keys yields a
normalised partial output and its log-sum-exp; the partials are merged by
weighting each with exp(lse_s - max_s lse_s).  The merge is the same
rescaling identity as the online update above, applied once across splits.
"""
import numpy as np


def _as_f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().double().numpy()
    except ImportError:
        pass
    return np.asarray(x, dtype=np.float64)


def _visible(Sq, Skv, causal, kv_len):
    """Boolean [Sq, Skv] mask of visible keys (bottom-right causal alignment)."""
    n = Skv if kv_len is None else max(0, min(Skv, int(kv_len)))
    j = np.arange(Skv)[None, :]
    i = np.arange(Sq)[:, None]
    vis = np.broadcast_to(j < n, (Sq, Skv))
    if causal:
        vis = vis & (j <= i + n - Sq)
    return vis


def online_attention(q, k, v, causal, scale, kv_lens=None, block_q=64, block_k=64):
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    o = np.zeros((B, Hq, Sq, d))
    for b in range(B):
        vis = _visible(Sq, Skv, causal, None if kv_lens is None else kv_lens[b])
        for h in range(Hq):
            g = h // group
            for i0 in range(0, Sq, block_q):
                qi = q[b, h, i0:i0 + block_q]
                rows = qi.shape[0]
                m = np.full(rows, -np.inf)
                l = np.zeros(rows)
                acc = np.zeros((rows, d))
                for j0 in range(0, Skv, block_k):
                    kj = k[b, g, j0:j0 + block_k]
                    vj = v[b, g, j0:j0 + block_k]
                    s = scale * (qi @ kj.T)
                    s = np.where(vis[i0:i0 + rows, j0:j0 + kj.shape[0]], s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    safe = np.where(np.isneginf(m_new), 0.0, m_new)
                    alpha = np.exp(m - safe)          # exp(-inf) = 0 when m was -inf
                    p = np.exp(s - safe[:, None])     # masked scores give 0
                    l = l * alpha + p.sum(axis=1)
                    acc = acc * alpha[:, None] + p @ vj
                    m = m_new
                nz = l > 0
                out = np.zeros((rows, d))
                out[nz] = acc[nz] / l[nz, None]
                o[b, h, i0:i0 + rows] = out
    return o


def partial(q_row, k_rows, v_rows, scale):
    """Normalised partial output and log-sum-exp of one query over a key subset."""
    if k_rows.shape[0] == 0:
        return np.zeros(q_row.shape[-1]), -np.inf
    s = scale * (k_rows @ q_row)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return (e @ v_rows) / l, m + np.log(l)


def combine(parts):
    """Merge (o_s, lse_s) partials by their log-sum-exp weights."""
    lses = np.array([p[1] for p in parts])
    if np.all(np.isneginf(lses)):
        return np.zeros_like(parts[0][0])
    mx = lses.max()
    w = np.exp(lses - mx)
    return sum(wi * p[0] for wi, p in zip(w, parts)) / w.sum()


def split_combine_attention(q, k, v, kv_lens, scale, boundaries):
    """Decode (one query row) with the keys cut at `boundaries` (a sorted list of
    split start positions, beginning with 0) and merged by combine()."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Sq, d = q.shape
    assert Sq == 1
    Hkv, Skv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    o = np.zeros((B, Hq, 1, d))
    for b in range(B):
        n = Skv if kv_lens is None else max(0, min(Skv, int(kv_lens[b])))
        edges = list(boundaries) + [Skv]
        for h in range(Hq):
            g = h // group
            parts = []
            for s0, s1 in zip(edges[:-1], edges[1:]):
                lo, hi = min(s0, n), min(s1, n)
                parts.append(partial(q[b, h, 0], k[b, g, lo:hi], v[b, g, lo:hi], scale))
            o[b, h, 0] = combine(parts)
    return o

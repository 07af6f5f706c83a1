"""Rotary position embedding before attention -- TEST INFRASTRUCTURE ONLY.

The pages name RoPE as a step that can run inside the attention kernel
("GPU learning day 24: Operator Fusion", section 6, the reference answer to
exercise 1; "What is kernel fusion and how is it used in LLM serving?",
section 3.5) but print no formula.  Reading used here: the rotary
embedding with rotate-half pairing.  For a vector x of even length d at
position p, with c_f = table[p, f] and s_f = table[p, d/2 + f] for
f < d/2 (the table holds cos(p * theta_f) and sin(p * theta_f)):

    y[f]       = x[f] * c_f - x[f + d/2] * s_f
    y[f + d/2] = x[f + d/2] * c_f + x[f] * s_f

i.e. each pair (x[f], x[f + d/2]) is rotated by the angle p * theta_f.
Positions: key j of a sequence sits at j; query i of a sequence with n
keys and S_q queries at n - S_q + i (the bottom-right alignment of the
causal mask), clamped at 0 for rows that see no key.

Everything is computed in float64 from the exact values of the inputs and
the table; the attention itself is the oracle's definition.
"""
import numpy as np

from . import attention as _attention


def _f64(x):
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:
        pass
    return np.asarray(x, dtype=np.float64)


def rope(x, table, positions):
    """Rotate the last axis of x [..., S, d] row by row: row i at positions[i]."""
    x = _f64(x)
    t = _f64(table)
    d = x.shape[-1]
    if d % 2 or t.shape[-1] != d:
        raise ValueError("x and the table need the same even last dimension")
    pos = np.asarray(positions, dtype=np.int64)
    if pos.shape != (x.shape[-2],) or pos.min(initial=0) < 0 or pos.max(initial=0) >= t.shape[0]:
        raise ValueError("one position per row, inside the table")
    h = d // 2
    c = t[pos, :h]                      # [S, d/2]
    s = t[pos, h:]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def positions(S_q, n):
    """Query positions n - S_q + i (clamped at 0) and key positions 0..n-1."""
    qpos = np.maximum(np.arange(S_q, dtype=np.int64) + n - S_q, 0)
    return qpos, np.arange(n, dtype=np.int64)


def attention_rope(q, k, v, causal, scale, table, kv_lens=None, lib=None):
    """fp64 attention of rope(q), rope(k), v over [B, H, S, d] inputs, with
    per-batch positions as above (kv_lens as in the oracle's attention; lib
    selects the evaluation as there)."""
    qf, kf = _f64(q), _f64(k)
    B, Hq, Sq, d = qf.shape
    Skv = kf.shape[2]
    lens = [Skv] * B if kv_lens is None else [max(0, min(Skv, int(x))) for x in kv_lens]
    qr = np.empty_like(qf)
    kr = np.empty_like(kf)
    for b in range(B):
        qpos, _ = positions(Sq, lens[b])
        qr[b] = rope(qf[b], table, qpos)
        kr[b] = rope(kf[b], table, np.arange(Skv, dtype=np.int64))
    return _attention(qr, kr, _f64(v), causal, scale, kv_lens=kv_lens, lib=lib)

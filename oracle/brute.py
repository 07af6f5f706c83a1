"""Scalar brute-force attention for tiny shapes -- TEST INFRASTRUCTURE ONLY.

An independent second route to the definition of attention ("GPU learning
day 24: Operator Fusion", section 3.4, standard attention): pure Python
floats, math.exp and math.fsum, one query row at a time, written separately
from oracle.c so that the two can pin each other.  Softmax here uses the
unshifted form exp(s_j) / sum exp(s_j) (no max subtraction), which is only
safe for the small scores of tiny test inputs; the C oracle's two-pass
max-shifted form must agree with it.

Inputs are nested lists (or anything indexable) of floats: q[b][h][i][c],
k[b][g][j][c], v[b][g][j][c].  The readings are the ones oracle.c states:
scale then mask, bottom-right causal alignment, KV head h // (Hq // Hkv),
kv_lens clamped to [0, S_kv], empty rows give 0.
"""
import math


def attention(q, k, v, causal, scale, kv_lens=None):
    B, Hq, Sq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv, Skv = len(k[0]), len(k[0][0])
    group = Hq // Hkv
    out = []
    for b in range(B):
        n_b = Skv if kv_lens is None else max(0, min(Skv, int(kv_lens[b])))
        ob = []
        for h in range(Hq):
            g = h // group
            oh = []
            for i in range(Sq):
                keys = [j for j in range(n_b) if (not causal) or j <= i + n_b - Sq]
                if not keys:
                    oh.append([0.0] * d)
                    continue
                w = [math.exp(scale * math.fsum(q[b][h][i][c] * k[b][g][j][c] for c in range(d)))
                     for j in keys]
                z = math.fsum(w)
                oh.append([math.fsum(w[t] * v[b][g][j][c] for t, j in enumerate(keys)) / z
                           for c in range(d)])
            ob.append(oh)
        out.append(ob)
    return out

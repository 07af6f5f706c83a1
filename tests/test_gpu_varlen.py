"""Packed variable-length prefill (attn_prefill_varlen_fwd) against the fp64
oracle per sequence, and bitwise against the padded-layout call when every
sequence has the same lengths."""
import numpy as np
import pytest
import torch

import attention_attn_fwd_11_amd as attn
import oracle
from attention_attn_fwd_11_amd import workloads as wl
from tests.gpu_util import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # Hq, Hkv, d, causal, q_lens, k_lens
    (8, 2, 128, True, [300, 1, 0, 700, 256, 513], [300, 5, 40, 700, 100, 1000]),
    (4, 4, 64, True, [1, 257, 640], [1, 257, 900]),
    (8, 1, 128, False, [77, 512, 3], [700, 64, 3]),
    (4, 2, 128, True, [200, 100], [0, 150]),                # a sequence with no key at all
    (4, 2, 256, True, [300, 129, 1], [400, 129, 2]),         # d = 256
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"H{c[0]}-{c[1]}-d{c[2]}-c{int(c[3])}-B{len(c[4])}")
def test_varlen_matches_oracle(case):
    Hq, Hkv, d, causal, q_lens, k_lens = case
    print(f"varlen {case}", flush=True)
    x = wl.varlen_problem(q_lens, k_lens, Hq, Hkv, d, device=DEV, seed=31)
    scale = 1.0 / np.sqrt(d)
    o = attn.prefill_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], max(q_lens), max(k_lens),
                            causal=causal, scale=scale)
    torch.cuda.synchronize()
    cq = x["cu_q"].tolist()
    ck = x["cu_k"].tolist()
    q, k, v, oc = x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), o.cpu()
    for b, (s, n) in enumerate(zip(q_lens, k_lens)):
        if s == 0:
            continue
        qb = q[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        kb = k[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        vb = v[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        got = oc[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0)
        if n == 0:
            assert torch.count_nonzero(got) == 0, f"sequence {b} has no key: O must be 0"
            continue
        ref = oracle.attention(qb, kb, vb, causal, scale)
        assert_close(got, ref, torch.bfloat16, f"varlen {case} sequence {b}")


@pytest.mark.parametrize("d", [128, 256])
def test_varlen_more_sequences_than_the_ranked_order_covers(d):
    """260 packed sequences (above the 256 the kernels rank longest first),
    some with no query or no key, against the oracle per sequence."""
    g = np.random.default_rng(80 + d)
    q_lens = [int(n) for n in g.integers(0, 50, size=260)]
    k_lens = [int(n) for n in g.integers(0, 60, size=260)]
    print(f"varlen 260 sequences d{d}", flush=True)
    x = wl.varlen_problem(q_lens, k_lens, 4, 2, d, device=DEV, seed=33)
    scale = 1.0 / np.sqrt(d)
    o = attn.prefill_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], max(q_lens), max(k_lens),
                            causal=True, scale=scale)
    torch.cuda.synchronize()
    cq, ck = x["cu_q"].tolist(), x["cu_k"].tolist()
    q, k, v, oc = x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), o.cpu()
    for b, (s, n) in enumerate(zip(q_lens, k_lens)):
        if s == 0:
            continue
        got = oc[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0)
        if n == 0:
            assert torch.count_nonzero(got) == 0, f"sequence {b} has no key: O must be 0"
            continue
        qb = q[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        kb = k[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        vb = v[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        ref = oracle.attention(qb, kb, vb, True, scale)
        assert_close(got, ref, torch.bfloat16, f"varlen 260 d{d} sequence {b}")


@pytest.mark.parametrize("causal", [True, False])
def test_varlen_equals_padded_for_equal_lengths(causal):
    B, Hq, Hkv, S, d = 3, 8, 2, 500, 128
    print(f"varlen vs padded causal={causal}", flush=True)
    x = wl.varlen_problem([S] * B, [S] * B, Hq, Hkv, d, device=DEV, seed=32)
    o = attn.prefill_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], S, S, causal=causal)
    pad = lambda t, H: t.view(B, S, H, d).permute(0, 2, 1, 3).contiguous()
    op = attn.prefill(pad(x["q"], Hq), pad(x["k"], Hkv), pad(x["v"], Hkv), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(pad(o, Hq), op)


def test_varlen_workload_sampled():
    w = wl.VARLEN
    lens = wl.kv_lengths(w).tolist()
    print(f"varlen workload {w.describe()} lens {lens}", flush=True)
    x = wl.varlen_problem(lens, lens, w.Hq, w.Hkv, w.d, device=DEV, seed=0)
    o = attn.prefill_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], max(lens), max(lens),
                            causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    cq = x["cu_q"].tolist()
    q, k, v, oc = x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), o.cpu()
    g = np.random.default_rng(3)
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), *map(int, g.choice(w.B, 3, replace=False))}):
        s = lens[b]
        qb = q[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        kb = k[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        vb = v[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        rows = sorted({(0, int(h), int(i)) for h, i in zip(g.integers(0, w.Hq, 40), g.integers(0, s, 40))}
                      | {(0, 0, 0), (0, w.Hq - 1, s - 1)})
        ref = oracle.attention_rows(qb, kb, vb, True, w.scale, rows)
        got = oc[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0)
        idx = torch.tensor(rows, dtype=torch.long)
        assert_close(got[idx[:, 0], idx[:, 1], idx[:, 2]], ref, torch.bfloat16, f"varlen workload seq {b}")

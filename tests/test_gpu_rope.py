"""Prefill with the rotary embedding (attn_prefill_rope_fwd), with K rotated
inside the attention kernel or once by a pre-pass into a workspace, against
the fp64 oracle that rotates Q and K first (oracle.rope).  Properties: both
K placements give identical bits; an identity table (cos 1, sin 0) gives
exactly the plain prefill's output; rotating Q and K on the host before a
plain prefill agrees to bf16 rounding; the pre-pass's rotated keys match
the oracle's rotation to one bf16 rounding and leave rows past kv_lens
alone."""
import sys

import numpy as np
import pytest
import torch

import attention_attn_fwd_11_amd as attn
import oracle
from attention_attn_fwd_11_amd import workloads as wl
from oracle import rope as orope
from tests.gpu_util import assert_close, convex_bound_ok, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def workspace(B, Hkv, S, d):
    n = attn.attn_prefill_rope_workspace_bytes(B, Hkv, S, d)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=DEV)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # B, Hq, Hkv, Sq, Skv, d, causal, kv_lens, extra table rows
    (2, 4, 2, 300, 300, 128, True, None, 0),
    (1, 4, 4, 700, 700, 64, True, None, 5),
    (2, 4, 1, 129, 1000, 128, True, None, 0),          # chunk of queries at the end of the keys
    (2, 2, 2, 200, 333, 128, False, None, 17),
    (3, 4, 2, 256, 600, 128, True, [600, 1, 300], 0),   # ragged KV lengths
    (2, 4, 2, 300, 300, 256, True, None, 0),
    (1, 2, 2, 100, 450, 256, False, [450], 3),
    (2, 4, 4, 64, 64, 64, False, [64, 0], 0),           # a sequence with no key
]


CASE_IDS = [f"B{c[0]}H{c[1]}-{c[2]}-q{c[3]}k{c[4]}-d{c[5]}-c{int(c[6])}-l{int(c[7] is not None)}"
            for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=CASE_IDS)
def test_rope_prefill_matches_oracle(case):
    """Both K placements against the oracle, and bit for bit against each other."""
    B, Hq, Hkv, Sq, Skv, d, causal, lens, spare = case
    say(f"rope prefill {case}")
    x = wl.random_problem(B, Hq, Hkv, Sq, Skv, d, dtype="bf16", device=DEV, seed=41)
    table = wl.rope_table(Skv + spare, d, device=DEV)
    scale = 1.0 / np.sqrt(d)
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=causal, scale=scale, kv_lens=lens_t, rope=table)
    o2 = attn.prefill(x["q"], x["k"], x["v"], causal=causal, scale=scale, kv_lens=lens_t, rope=table,
                      rope_workspace=workspace(B, Hkv, Skv, d))
    torch.cuda.synchronize()
    ref = orope.attention_rope(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), causal, scale, table.cpu(),
                               kv_lens=lens)
    assert_close(o, ref, torch.bfloat16, f"rope prefill {case}")
    assert torch.equal(o, o2), "K rotated in the kernel and by the pre-pass must give the same bits"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rope_prepass_keys(d):
    """The workspace holds rope(K) (the oracle's fp64 rotation, one bf16
    rounding apart) for rows below kv_lens and is untouched past them."""
    say(f"rope pre-pass keys d{d}")
    B, Hkv, S = 3, 2, 300
    x = wl.random_problem(B, Hkv, Hkv, 4, S, d, dtype="bf16", device=DEV, seed=44)
    table = wl.rope_table(S + 9, d, theta=300.0, device=DEV)
    lens = [300, 17, 0]
    ws = workspace(B, Hkv, S, d)
    ws.fill_(0x7f)                                  # bf16 0x7f7f: a large finite sentinel
    attn.prefill(x["q"], x["k"], x["v"], causal=True, kv_lens=torch.tensor(lens, dtype=torch.int32,
                 device=DEV), rope=table, rope_workspace=ws)
    torch.cuda.synchronize()
    kr = ws[: B * Hkv * S * d * 2].view(torch.bfloat16).view(B, Hkv, S, d).cpu()
    ref = orope.rope(x["k"].cpu(), table.cpu(), np.arange(S))
    sentinel = torch.tensor([0x7f7f], dtype=torch.int16).view(torch.bfloat16)[0]
    for b, n in enumerate(lens):
        got = kr[b, :, :n].double().numpy()
        want = ref[b, :, :n]
        # fp32 products and an fma (error ~2^-23 of |x1| + |x2|, which matters
        # only where the two terms cancel), then one rounding to bf16 (half
        # an ulp, at most 2^-8 of the value)
        mag = float(np.abs(x["k"][b].float().cpu().numpy()).max())
        tol = 2.0 ** -8 * np.abs(want) + 2.0 ** -20 * mag
        assert np.all(np.abs(got - want) <= tol), f"batch {b}: {np.abs(got - want).max():.3g}"
        assert bool((kr[b, :, n:] == sentinel).all()), f"batch {b}: rows past kv_lens written"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_identity_table_equals_plain_prefill(d):
    say(f"rope identity table d{d}")
    B, Hq, Hkv, S = 2, 4, 2, 333
    x = wl.random_problem(B, Hq, Hkv, S, S, d, dtype="bf16", device=DEV, seed=42)
    table = torch.cat([torch.ones(S, d // 2), torch.zeros(S, d // 2)], dim=1).to(DEV)
    a = attn.prefill(x["q"], x["k"], x["v"], causal=True, rope=table)
    a2 = attn.prefill(x["q"], x["k"], x["v"], causal=True, rope=table,
                      rope_workspace=workspace(B, Hkv, S, d))
    b = attn.prefill(x["q"], x["k"], x["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, a2), "K rotated in the kernel and by the pre-pass must give the same bits"
    if d < 256:
        # the rotary and the plain calls run the same kernel: bit equality
        assert torch.equal(a, b), "cos 1 / sin 0 must leave Q and K unchanged"
    else:
        # at d = 256 the plain call runs the 16-row kernel, the rotary calls the
        # 32-row one (different summation orders): both against the definition
        ref = oracle.attention(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), True, 1.0 / np.sqrt(d))
        assert_close(a, ref, torch.bfloat16, "rope identity table d256")
        assert_close(b, ref, torch.bfloat16, "plain d256")


def test_rope_equals_host_rotation_then_plain_prefill():
    """Rotating Q and K on the host (fp64, rounded to bf16 once) and then
    running the plain prefill must agree with the fused path to bf16
    rounding: the fused path rounds the same rotated values once too."""
    say("rope vs host rotation")
    B, Hq, Hkv, S, d = 1, 4, 2, 520, 128
    x = wl.random_problem(B, Hq, Hkv, S, S, d, dtype="bf16", device=DEV, seed=43)
    table = wl.rope_table(S, d, theta=500.0, device=DEV)
    pos = np.arange(S)
    qr = torch.from_numpy(orope.rope(x["q"].cpu(), table.cpu(), pos)).to(torch.bfloat16).to(DEV)
    kr = torch.from_numpy(orope.rope(x["k"].cpu(), table.cpu(), pos)).to(torch.bfloat16).to(DEV)
    fused = attn.prefill(x["q"], x["k"], x["v"], causal=True, rope=table)
    host = attn.prefill(qr, kr, x["v"], causal=True)
    torch.cuda.synchronize()
    diff = (fused.float() - host.float()).abs()
    assert float(diff.max()) <= 1e-2 and float(diff.mean()) <= 1e-3, \
        f"fused vs host rotation: max {float(diff.max()):.3e} mean {float(diff.mean()):.3e}"


def test_rope_workload_sampled():
    """The headline causal shape (B 4, H 32, S 4096, d 128) with RoPE:
    sampled rows against the oracle, whole output inside V's convex hull."""
    w = wl.BY_NAME["prefill_bf16_b4h32s4096"]
    say(f"rope workload: {w.describe()}")
    x = wl.generate(w, DEV)
    table = wl.rope_table(w.Skv, w.d, device=DEV)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=True, scale=w.scale, rope=table)
    o2 = attn.prefill(x["q"], x["k"], x["v"], causal=True, scale=w.scale, rope=table,
                      rope_workspace=workspace(w.B, w.Hkv, w.Skv, w.d))
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "K placements differ at the full size"
    ok, finite = convex_bound_ok(o, x["v"], w.Hq)
    assert finite and ok, "output outside the convex hull of V"
    S = w.Sq
    rows = sample_rows(w.B, w.Hq, S, 120, seed=2, extra=[(0, 0, 0), (w.B - 1, w.Hq - 1, S - 1),
                                                          (1, 5, 255), (2, 7, 256)])
    pos = np.arange(S)
    tc = table.cpu()
    qr = orope.rope(x["q"].cpu(), tc, pos)
    kr = orope.rope(x["k"].cpu(), tc, pos)
    ref = oracle.attention_rows(qr, kr, x["v"].cpu().double(), True, w.scale, rows)
    idx = torch.tensor(rows, dtype=torch.long)
    got = o[idx[:, 0], idx[:, 1], idx[:, 2]]
    assert_close(got, ref, torch.bfloat16, "rope headline sampled rows")

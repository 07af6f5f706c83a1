"""Edge cases of the scale: a negative scale (the bf16 prefill then takes
the row minimum of the raw scores as its reference, a template instance of
its own) on every entry point, and scales so large that each row's softmax
is nearly one-hot (exponents far below exp2's range, the lazy rescale
crossing its threshold on many blocks).  All against the fp64 oracle."""
import sys

import numpy as np
import pytest
import torch

import attention_attn_fwd_11_amd as attn
import oracle
from attention_attn_fwd_11_amd import workloads as wl
from oracle import rope as orope
from tests.gpu_util import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def lens_t(lens):
    return None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)


PREFILL = [
    # B, Hq, Hkv, Sq, Skv, d, causal, lens, dtype
    (2, 4, 2, 300, 300, 128, True, None, "bf16"),
    (2, 4, 4, 130, 330, 128, False, [330, 17], "bf16"),
    (1, 8, 8, 530, 530, 64, True, None, "bf16"),
    (2, 4, 2, 200, 330, 256, True, [330, 0], "bf16"),
    (2, 4, 2, 200, 260, 128, True, [260, 100], "f32"),
]


@pytest.mark.parametrize("scale_mult", [-1.0, 6.0, -6.0])
@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}-{c[8]}")
def test_prefill_scale_edges(case, scale_mult):
    B, Hq, Hkv, Sq, Skv, d, causal, lens, dtype = case
    scale = scale_mult / np.sqrt(d)
    say(f"prefill {case} scale {scale:.4f}")
    x = wl.random_problem(B, Hq, Hkv, Sq, Skv, d, dtype=dtype, device=DEV, seed=51)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=causal, scale=scale, kv_lens=lens_t(lens))
    torch.cuda.synchronize()
    ref = oracle.attention(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), causal, scale, kv_lens=lens)
    assert_close(o, ref, torch.float32 if dtype == "f32" else torch.bfloat16,
                 f"prefill {case} scale {scale}")


@pytest.mark.parametrize("scale_mult", [-1.0, 6.0])
@pytest.mark.parametrize("B,Hq,Hkv,S,d,lens", [(3, 4, 4, 1100, 128, [1100, 513, 0]),
                                              (3, 8, 2, 900, 128, [900, 128, 257]),
                                              (2, 4, 4, 700, 64, [700, 5])],
                         ids=["mha", "gqa", "mha-d64"])
def test_decode_scale_edges(B, Hq, Hkv, S, d, lens, scale_mult):
    scale = scale_mult / np.sqrt(d)
    say(f"decode B{B} Hq{Hq} Hkv{Hkv} S{S} d{d} scale {scale:.4f}")
    x = wl.random_problem(B, Hq, Hkv, 1, S, d, dtype="bf16", device=DEV, seed=52)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_t(lens), scale=scale)
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, scale)
    assert_close(o, ref, torch.bfloat16, f"decode scale {scale}")


@pytest.mark.parametrize("scale_mult", [-1.0, 6.0])
def test_varlen_scale_edges(scale_mult):
    q_lens, k_lens = [300, 1, 700], [300, 40, 900]
    Hq, Hkv, d = 8, 2, 128
    scale = scale_mult / np.sqrt(d)
    say(f"varlen scale {scale:.4f}")
    x = wl.varlen_problem(q_lens, k_lens, Hq, Hkv, d, device=DEV, seed=53)
    o = attn.prefill_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], max(q_lens), max(k_lens),
                            causal=True, scale=scale)
    torch.cuda.synchronize()
    cq, ck = x["cu_q"].tolist(), x["cu_k"].tolist()
    q, k, v, oc = x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), o.cpu()
    for b in range(len(q_lens)):
        qb = q[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        kb = k[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        vb = v[ck[b]:ck[b + 1]].permute(1, 0, 2).unsqueeze(0).contiguous()
        got = oc[cq[b]:cq[b + 1]].permute(1, 0, 2).unsqueeze(0)
        ref = oracle.attention(qb, kb, vb, True, scale)
        assert_close(got, ref, torch.bfloat16, f"varlen sequence {b} scale {scale}")


@pytest.mark.parametrize("prepass", [False, True], ids=["k-in-kernel", "k-prepass"])
def test_rope_negative_scale(prepass):
    B, Hq, Hkv, S, d = 2, 4, 2, 333, 128
    scale = -1.0 / np.sqrt(d)
    say(f"rope negative scale prepass={prepass}")
    x = wl.random_problem(B, Hq, Hkv, S, S, d, dtype="bf16", device=DEV, seed=54)
    table = wl.rope_table(S, d, device=DEV)
    ws = None
    if prepass:
        ws = torch.empty(attn.attn_prefill_rope_workspace_bytes(B, Hkv, S, d), dtype=torch.uint8,
                         device=DEV)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=True, scale=scale, rope=table, rope_workspace=ws)
    torch.cuda.synchronize()
    ref = orope.attention_rope(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), True, scale, table.cpu())
    assert_close(o, ref, torch.bfloat16, "rope negative scale")

"""The LDS-poison debug build (libattn_lds_poison.so) on the GPU.

In that build every direct global -> LDS copy first fills its destination
with bf16 NaNs and waits for the fill, so a read of a staging buffer that is
not ordered after its copy by the kernel's waits and barriers returns NaN
instead of the previous tile.  Each kernel that stages K/V by direct copies
(the bf16 prefill at d = 64 and 128, causal pairs, RoPE and packed
sequences; the d = 256 prefill; the balanced GQA decode, contiguous and
paged) runs here on shapes with several stages, ragged tails and empty
sequences.  The poison is always overwritten before a correctly ordered read,
so the outputs must equal the normal build's bit for bit, and they must match
the fp64 oracle within the bf16 bar.
"""
import os
import sys

import numpy as np
import pytest
import torch

import attention_attn_fwd_11_amd as attn
import oracle
from attention_attn_fwd_11_amd import workloads as wl
from tests.gpu_util import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(attn.lds_poison_library_path), "libattn_lds_poison.so must be built"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def both(fn):
    """fn() on the normal build, then on the poison build; both outputs."""
    a = fn()
    torch.cuda.synchronize()
    with attn.use_library(attn.lds_poison_library_path):
        b = fn()
        torch.cuda.synchronize()
    return a, b


PREFILL = [
    # B, Hq, Hkv, S_q, S_kv, d, causal, lens
    (2, 8, 2, 520, 777, 128, True, [777, 300]),
    (1, 4, 2, 1100, 1100, 128, True, None),
    (1, 8, 8, 700, 640, 128, False, [640]),
    (1, 16, 8, 530, 530, 64, True, None),
    (2, 4, 1, 130, 700, 256, True, [700, 257]),
    (1, 8, 8, 600, 600, 256, True, None),
    (3, 4, 2, 150, 260, 64, True, [260, 97, 0]),
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}")
def test_prefill_poison_build_matches(case):
    B, Hq, Hkv, Sq, Skv, d, causal, lens = case
    say(f"lds-poison prefill {case}")
    x = wl.random_problem(B, Hq, Hkv, Sq, Skv, d, dtype="bf16", device=DEV, seed=11)
    scale = 1.0 / np.sqrt(d)
    lt = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    a, b = both(lambda: attn.prefill(x["q"], x["k"], x["v"], causal=causal, scale=scale, kv_lens=lt))
    assert torch.equal(a, b), "poison build differs from the normal build"
    ref = oracle.attention(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), causal, scale, kv_lens=lens)
    assert_close(b, ref, torch.bfloat16, f"lds-poison prefill {case}")


def test_prefill_rope_poison_build_matches():
    from oracle.rope import attention_rope
    B, H, S, d = 1, 4, 600, 128
    say(f"lds-poison rope prefill B{B} H{H} S{S} d{d}")
    x = wl.random_problem(B, H, H, S, S, d, dtype="bf16", device=DEV, seed=12)
    table = wl.rope_table(S, d).to(DEV)
    scale = 1.0 / np.sqrt(d)
    a, b = both(lambda: attn.prefill(x["q"], x["k"], x["v"], causal=True, scale=scale, rope=table))
    assert torch.equal(a, b), "poison build differs from the normal build"
    ref = attention_rope(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), True, scale, table.cpu())
    assert_close(b, ref, torch.bfloat16, "lds-poison rope prefill")


def test_prefill_varlen_poison_build_matches():
    q_lens, k_lens = [300, 1, 0, 650], [300, 90, 5, 650]
    Hq, Hkv, d = 4, 2, 128
    say(f"lds-poison varlen prefill q{q_lens} k{k_lens}")
    p = wl.varlen_problem(q_lens, k_lens, Hq, Hkv, d, device=DEV, seed=13)
    scale = 1.0 / np.sqrt(d)
    a, b = both(lambda: attn.prefill_varlen(p["q"], p["k"], p["v"], p["cu_q"], p["cu_k"], max(q_lens),
                                             max(k_lens), causal=True, scale=scale))
    assert torch.equal(a, b), "poison build differs from the normal build"


DECODE = [
    # B, Hq, Hkv, S_cap, d, lens   (query groups: the balanced pass)
    (4, 8, 2, 700, 128, [700, 256, 255, 3]),
    (3, 4, 2, 1100, 128, [513, 767, 1024]),
    (5, 32, 8, 1500, 128, [1500, 1, 0, 900, 129]),
    (3, 8, 1, 900, 64, [2, 900, 0]),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "x".join(map(str, c[:5])))
def test_decode_poison_build_matches(case):
    B, Hq, Hkv, S, d, lens = case
    say(f"lds-poison decode {case}")
    x = wl.random_problem(B, Hq, Hkv, 1, S, d, dtype="bf16", device=DEV, seed=14)
    scale = 1.0 / np.sqrt(d)
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    a, b = both(lambda: attn.decode(x["q"], x["k"], x["v"], kv_lens=lt, scale=scale))
    assert torch.equal(a, b), "poison build differs from the normal build"
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, scale)
    assert_close(b, ref, torch.bfloat16, f"lds-poison decode {case}")
    # the paged cache runs the same kernel with page-table addressing
    kp, vp, table = wl.paged_cache(x["k"], x["v"], lens, 256, seed=15)
    c, e = both(lambda: attn.decode_paged(x["q"], kp, vp, table, kv_lens=lt, scale=scale))
    assert torch.equal(c, e), "paged: poison build differs from the normal build"
    assert torch.equal(c, a), "paged and contiguous decode differ"

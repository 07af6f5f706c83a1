"""The allocation-free decode (attn_decode_noalloc_fwd) against the decode
that takes a caller's workspace (attn_decode_fwd), both through the C ABI:
two calls in a row on one GPU, the second smaller, for one query head per
KV head (chunked split pass), for query groups (balanced pass) and for an
fp32 cache.  The kernels are the same, so the outputs must be bitwise
equal; the first call is also held to the dtype's bar against the fp64
oracle."""
import ctypes
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
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def run_both(x, lens, scale, dt):
    q, k, v = x["q"], x["k"], x["v"]
    B, Hq, _, d = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o_static = torch.full_like(q, float("nan"))
    st = attn.attn_decode_noalloc_fwd(ptr(q), ptr(k), ptr(v), ptr(o_static), B, Hq, Hkv, 1, S, d, 0,
                                      scale, ptr(lens), dt, stream)
    assert st == 0, attn.attn_status_str(st)
    need = attn.attn_decode_workspace_bytes(B, Hq, Hkv, S, d)
    assert need <= attn.ATTN_DECODE_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    o_ws = torch.full_like(q, float("nan"))
    st = attn.attn_decode_fwd(ptr(q), ptr(k), ptr(v), ptr(o_ws), B, Hq, Hkv, 1, S, d, 0, scale,
                              ptr(lens), dt, ptr(ws), need, stream)
    assert st == 0, attn.attn_status_str(st)
    torch.cuda.synchronize()
    return o_static, o_ws


@pytest.mark.parametrize("Hq,Hkv,dtype", [(32, 32, "bf16"), (32, 8, "bf16"), (12, 4, "f32")],
                         ids=["mha-chunked", "gqa-balanced", "f32-group3"])
def test_noalloc_decode_matches_workspace_decode(Hq, Hkv, dtype):
    d = 128
    scale = 1.0 / np.sqrt(d)
    # first call: ragged lengths up to 4096 over 24 sequences; second: smaller
    for call, (B, S, seed) in enumerate([(24, 4096, 71), (5, 700, 72)]):
        say(f"noalloc decode call {call}: B{B} Hq{Hq} Hkv{Hkv} S{S} {dtype}")
        x = wl.random_problem(B, Hq, Hkv, 1, S, d, dtype=dtype, device=DEV, seed=seed)
        g = torch.Generator().manual_seed(seed)
        lens = torch.randint(0, S + 1, (B,), generator=g, dtype=torch.int32)
        lens[0] = S
        o_static, o_ws = run_both(x, lens.to(DEV), scale, attn.ATTN_F32 if dtype == "f32" else attn.ATTN_BF16)
        assert torch.equal(o_static, o_ws), f"call {call}: allocation-free decode differs"
        if call == 0:
            ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens.tolist(), scale)
            assert_close(o_static, ref, torch.float32 if dtype == "f32" else torch.bfloat16,
                         f"noalloc call {call}")

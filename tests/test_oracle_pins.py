"""The oracle checked against its pins (CPU only).

Both evaluations of the definition are pinned: the scalar one in oracle.c
and the row-block one with library matrix products (oracle/rowblock.py),
which the full-size GPU parity tests use.
"""
import numpy as np
import pytest

import oracle
from oracle import rowblock
from tests import oracle_pins


@pytest.fixture(scope="module", params=["oracle_c", "rowblock"])
def lib(request):
    return oracle.load() if request.param == "oracle_c" else rowblock


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)


@pytest.mark.parametrize("fn", ["attention", "attention_rows"])
def test_mixed_input_dtypes_rejected(fn, lib):
    """q, k and v are read in one stored format: mixing them is an error,
    not a read of one array in another's element size."""
    q = np.zeros((1, 1, 4, 8))
    kv = np.zeros((1, 1, 4, 8), np.float32)
    call = getattr(oracle, fn)
    args = (q, q, kv, True, 0.5) + (([(0, 0, 1)],) if fn == "attention_rows" else ())
    with pytest.raises(TypeError):
        call(*args, lib=lib)


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, Sq, Skv, d, causal, kv_lens, kscale
    (2, 4, 2, 300, 300, 128, True, None, 1.0),
    (2, 4, 2, 130, 700, 64, True, [700, 257], 4.0),
    (1, 4, 4, 600, 330, 128, False, [330], 1.0),
    (3, 4, 1, 300, 260, 64, True, [260, 97, 0], 1.0),
    (2, 8, 2, 1, 900, 128, False, [900, 31], 4.0),
])
def test_rowblock_equals_scalar_oracle(case):
    """The two evaluations agree to rounding on shapes that span several row
    blocks, ragged lengths, empty sequences, GQA and the decode shape."""
    import torch
    B, Hq, Hkv, Sq, Skv, d, causal, lens, ks = case
    g = torch.Generator().manual_seed(11)
    q = torch.randn(B, Hq, Sq, d, generator=g).to(torch.bfloat16)
    k = (torch.randn(B, Hkv, Skv, d, generator=g) * ks).to(torch.bfloat16)
    v = torch.randn(B, Hkv, Skv, d, generator=g).to(torch.bfloat16)
    a, la = oracle.attention(q, k, v, causal, d ** -0.5, kv_lens=lens, want_lse=True)
    b, lb = oracle.attention(q, k, v, causal, d ** -0.5, kv_lens=lens, want_lse=True, lib=rowblock)
    assert np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.max(np.abs(a)))
    fin = np.isfinite(la)
    assert np.array_equal(fin, np.isfinite(lb))
    assert np.max(np.abs(la[fin] - lb[fin]), initial=0.0) <= 1e-12 * max(1.0, np.max(np.abs(la[fin]), initial=0))

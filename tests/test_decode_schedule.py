"""Host model of the balanced decode pass's work split and partial slots,
checked against the sizes the C ABI reports (no GPU).

The pass cuts every (sequence, virtual KV head) into units of 128 keys,
ordered (sequence, head, unit); workgroup w takes the contiguous units
[w*R, (w+1)*R) with R = ceil(U / workgroups) and writes one partial per
run, a maximal part of its range inside one head, at slot head + u0 / R
(u0: the run's first unit).  The combine reads, for each head with units
[hs, he), the slots head + hs/R .. head + (he-1)/R.  This model enumerates
the runs the workgroups produce and checks that:
  - every head's runs occupy exactly that contiguous slot range, once each;
  - no two runs of different heads share a slot;
  - every slot lies below the partial rows attn_decode_workspace_bytes
    provides (per column of a query block).
"""
import math
import os

import numpy as np
import pytest

import attention_attn_fwd_11_amd as attn

UNIT = 128          # keys per unit
MAX_WG = 1024       # most workgroups of the pass


def runs(units_per_head, n_wg):
    """(head, first unit) of every run the workgroups produce."""
    U = sum(units_per_head)
    if U == 0:
        return [], 1
    R = -(-U // n_wg)
    starts = np.concatenate([[0], np.cumsum(units_per_head)])
    out = []
    for w in range(n_wg):
        u, end = w * R, min((w + 1) * R, U)
        while u < end:
            h = int(np.searchsorted(starts, u, side="right") - 1)
            seg_end = min(end, int(starts[h + 1]))
            out.append((h, u))
            u = seg_end
    return out, R


def check(units_per_head, n_wg):
    out, R = runs(units_per_head, n_wg)
    starts = np.concatenate([[0], np.cumsum(units_per_head)])
    slots = {}
    for h, u in out:
        s = h + u // R
        assert s not in slots, f"slot {s} written twice"
        slots[s] = h
    for h, n in enumerate(units_per_head):
        hs, he = int(starts[h]), int(starts[h]) + n
        mine = sorted(s for s, hh in slots.items() if hh == h)
        expect = list(range(h + hs // R, h + (he - 1) // R + 1)) if n else []
        assert mine == expect, f"head {h}: runs at {mine}, combine reads {expect}"
    return max(slots) + 1 if slots else 0


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.library_path):
        pytest.skip("libattn.so not built (run __graft_entry__.build())")
    return attn._load()


@pytest.mark.parametrize("seed", range(40))
def test_runs_fill_the_slots_the_combine_reads(seed):
    g = np.random.default_rng(seed)
    heads = int(g.integers(1, 300))
    units = [int(x) for x in g.integers(0, 70, heads)]
    if g.random() < 0.3:
        units = [u if g.random() < 0.7 else 0 for u in units]   # empty sequences
    n_wg = int(g.choice([1, 3, 7, 256, 512, 1024, 100000]))
    n_wg = min(n_wg, max(sum(units), 1), MAX_WG)
    used = check(units, n_wg)
    assert used <= heads + n_wg


@pytest.mark.parametrize("B,Hq,Hkv,S,d", [(128, 32, 8, 8192, 128), (3, 40, 2, 20000, 256),
                                          (2048, 4, 1, 40, 128), (1, 8, 1, 131072, 64)])
def test_slots_fit_the_workspace(lib, B, Hq, Hkv, S, d):
    """Full-length sequences (the most units): the highest slot the model
    reaches, times the column block, fits the rows the workspace holds."""
    G = Hq // Hkv
    blocks = -(-G // 16)
    cb = -(-G // blocks)
    hv = Hkv * blocks
    units = [math.ceil(S / UNIT)] * (B * hv)
    n_wg = min(512, sum(units), MAX_WG)
    used = check(units, n_wg)
    ws = attn.attn_decode_workspace_bytes(B, Hq, Hkv, S, d)
    assert ws > 0
    rows = used * cb
    assert rows * d * 4 + rows * 4 <= ws, (rows, ws)

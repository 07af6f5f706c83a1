"""Pins from the one worked number the pages print for attention.

tests/golden/score_matrix_s4096_fp16.json restates the score-matrix size
that "GPU learning day 24: Operator Fusion", section 3.4, works out for
S = 4096 in fp16 and how often unfused attention moves it.  The fused path
must never move that matrix: the HBM write traffic measured for the
headline prefill (rocprofv3 WRITE_SIZE, calibrated, in profiles/traffic.json)
has to be the output O alone.
"""
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "score_matrix_s4096_fp16.json")
TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_page_arithmetic():
    g = golden()
    assert g["S"] * g["S"] * g["bytes_per_element"] == g["matrix_bytes"] == 32 * 2**20
    assert (g["writes"], g["reads"]) == (1, 3)


def test_measured_prefill_writes_hold_no_score_matrix():
    g = golden()
    with open(TRAFFIC) as f:
        t = json.load(f)["workloads"]["prefill_bf16_b4h32s4096"]
    B, H, S, d = 4, 32, 4096, 128
    assert S == g["S"]
    out_bytes = B * H * S * d * 2                      # O in bf16
    unfused_writes = B * H * g["writes"] * g["matrix_bytes"]
    unfused_moves = B * H * (g["writes"] + g["reads"]) * g["matrix_bytes"]
    assert unfused_writes == 4 * 2**30 and unfused_moves == 16 * 2**30
    # what the fused kernel wrote is O, to within 1 % (no S x S term)
    assert abs(t["write_bytes_per_launch"] - out_bytes) <= 0.01 * out_bytes
    assert t["write_bytes_per_launch"] < 0.05 * unfused_writes
    # everything it moved is less than a tenth of the score traffic alone
    assert t["hbm_bytes_per_launch"] < 0.1 * unfused_moves

"""The recorded HBM traffic of the fused kernels (profiles/traffic.json,
rocprofv3 FETCH_SIZE and WRITE_SIZE, calibrated against a copy of known
size) against what the pages fix (CPU only).

"Optimizing Decoder Attention for LLMs on GPU", fused kernels and a single
kernel: in the fused decode each K and V element is read from global memory
once per step.  Both decodes' measured reads must be the visible K/V bytes
within 1 %.  "GPU learning day 24: Operator Fusion", section 3.4: the fused
prefill writes only O (no score matrix) -- writes within 1 % of |O|.
"""
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REC = os.path.join(ROOT, "profiles", "traffic.json")


@pytest.fixture(scope="module")
def rec():
    with open(REC) as f:
        return json.load(f)["workloads"]


@pytest.mark.parametrize("name", ["decode_bf16_b64h32l4096", "decode_gqa_bf16_b128h32kv8"])
def test_decode_reads_each_kv_byte_once(rec, name):
    from attention_attn_fwd_11_amd import workloads as wl
    r = rec[name]
    w = wl.BY_NAME[name]
    alg = wl.decode_kv_bytes(w, wl.kv_lengths(w))
    assert r["min_read_bytes"] == alg
    assert abs(r["fetch_bytes_per_launch"] / alg - 1.0) <= 0.01, \
        f"{name}: read {r['fetch_bytes_per_launch']} B for {alg} B of visible K/V"


@pytest.mark.parametrize("name", ["prefill_bf16_b4h32s4096", "prefill_gqa_bf16_h64kv8s16384"])
def test_prefill_writes_only_o(rec, name):
    from attention_attn_fwd_11_amd import workloads as wl
    w = wl.BY_NAME[name]
    o_bytes = w.B * w.Hq * w.Sq * w.d * 2
    assert rec[name]["min_write_bytes"] == o_bytes
    assert abs(rec[name]["write_bytes_per_launch"] / o_bytes - 1.0) <= 0.01

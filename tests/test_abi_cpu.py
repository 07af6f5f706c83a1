"""C ABI checks that need no GPU: the library loads, exports every function
include/attn.h declares, and rejects invalid arguments on the host before
any HIP call (so no kernel is ever launched here)."""
import ctypes
import math
import os
import re

import pytest

import attention_attn_fwd_11_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

NULL = None
P = ctypes.c_void_p(0x10000)       # a 16-byte aligned dummy address, never dereferenced
MIS = ctypes.c_void_p(0x10008)     # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(attn.library_path):
        pytest.skip("libattn.so not built (run __graft_entry__.build())")
    return attn._load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"attn_prefill_fwd", "attn_prefill_rope_fwd", "attn_prefill_rope_workspace_bytes",
            "attn_prefill_varlen_fwd", "attn_decode_fwd",
            "attn_decode_paged_fwd", "attn_decode_noalloc_fwd",
            "attn_decode_workspace_bytes", "attn_status_str", "attn_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libattn.so does not export {n}"


def test_status_strings(lib):
    for code in range(0, 8):
        s = attn.attn_status_str(code)
        assert s and s != "unknown status"
    assert attn.attn_status_str(99) == "unknown status"


def prefill(q=P, k=P, v=P, o=P, B=1, Hq=2, Hkv=2, Sq=8, Skv=8, d=64, causal=1, scale=0.125,
            lens=NULL, dtype=attn.ATTN_BF16):
    return attn.attn_prefill_fwd(q, k, v, o, B, Hq, Hkv, Sq, Skv, d, causal, scale, lens, dtype,
                                 NULL)


def decode(q=P, k=P, v=P, o=P, B=1, Hq=2, Hkv=2, Sq=1, Skv=8, d=64, causal=0, scale=0.125,
           lens=NULL, dtype=attn.ATTN_BF16, ws=P, wsb=1 << 30):
    return attn.attn_decode_fwd(q, k, v, o, B, Hq, Hkv, Sq, Skv, d, causal, scale, lens, dtype, ws,
                                wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(k=NULL), 1), (dict(v=NULL), 1), (dict(o=NULL), 1),
    (dict(B=-1), 2), (dict(Sq=-1), 2), (dict(Skv=-2), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2),
    (dict(Hq=6, Hkv=4), 2), (dict(causal=2), 2), (dict(Sq=9, Skv=8, causal=1), 2),
    (dict(d=96), 3), (dict(d=512), 3), (dict(dtype=5), 3),
    (dict(q=MIS), 4), (dict(o=MIS), 4), (dict(k=MIS), 4), (dict(v=MIS), 4),
    (dict(scale=math.inf), 7), (dict(scale=math.nan), 7),
    # one head's rows must span at most 2^31 - 1 bytes
    (dict(Skv=(1 << 23) + 1, d=128), 2), (dict(Sq=(1 << 23) + 1, Skv=(1 << 23) + 1, causal=0, d=128), 2),
    (dict(Skv=(1 << 22) + 1, d=128, dtype=attn.ATTN_F32), 2),
    (dict(Skv=(1 << 21) + 1, d=256, dtype=attn.ATTN_F32), 2),
    # B * H_q at most 2^30 - 1; fp32 indexes B and H_q by grid dimensions of at most 65535
    (dict(B=1 << 15, Hq=1 << 15, Hkv=1 << 15), 2),
    (dict(B=65536, Hq=1, Hkv=1, dtype=attn.ATTN_F32), 2), (dict(B=1, Hq=65536, Hkv=1, dtype=attn.ATTN_F32), 2),
])
def test_prefill_rejects(lib, kw, code):
    assert prefill(**kw) == code


def test_prefill_empty_is_noop(lib):
    # nothing to compute: succeeds without touching the device
    assert prefill(q=NULL, o=NULL, B=0) == 0
    assert prefill(q=NULL, o=NULL, Sq=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(o=NULL), 1), (dict(k=NULL), 1),
    (dict(Sq=2), 2), (dict(Sq=0), 2), (dict(Hq=6, Hkv=4), 2), (dict(B=-3), 2),
    (dict(dtype=attn.ATTN_F32, d=96), 3), (dict(dtype=9), 3),
    (dict(d=32), 3), (dict(d=512), 3),
    (dict(ws=NULL), 5), (dict(wsb=16), 5), (dict(ws=MIS), 4), (dict(k=MIS), 4),
    (dict(scale=-math.inf), 7), (dict(Skv=(1 << 23) + 1, d=128), 2),
    # batches and query heads are grid dimensions of at most 65535
    (dict(B=65536, Hq=1, Hkv=1), 2), (dict(B=1, Hq=65536, Hkv=65536), 2),
    (dict(B=65536, Hq=1, Hkv=1, dtype=attn.ATTN_F32), 2),
])
def test_decode_rejects(lib, kw, code):
    assert decode(**kw) == code


def decode_noalloc(q=P, k=P, v=P, o=P, B=1, Hq=2, Hkv=2, Sq=1, Skv=8, d=64, causal=0, scale=0.125,
                   lens=NULL, dtype=attn.ATTN_BF16):
    return attn.attn_decode_noalloc_fwd(q, k, v, o, B, Hq, Hkv, Sq, Skv, d, causal, scale, lens,
                                        dtype, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(o=NULL), 1), (dict(k=NULL), 1),
    (dict(Sq=2), 2), (dict(Hq=6, Hkv=4), 2), (dict(B=-3), 2),
    (dict(dtype=attn.ATTN_F32, d=96), 3), (dict(dtype=9), 3),
    (dict(d=32), 3), (dict(d=512), 3),
    (dict(q=MIS), 4), (dict(scale=math.nan), 7),
    # partials beyond the static scratch: B*H_q chunked splits of (d + 1) floats
    (dict(B=2048, Hq=32, Hkv=32, Skv=4096, d=128), 5),
    (dict(B=65536, Hq=1, Hkv=1), 2),
])
def test_decode_noalloc_rejects(lib, kw, code):
    """The allocation-free decode validates on the host, before it looks up
    its scratch, and refuses sizes whose partials exceed the scratch."""
    assert decode_noalloc(**kw) == code


def test_decode_noalloc_scratch_limit(lib):
    """The workloads' decodes fit the static scratch; the rejected shape above
    does not."""
    lim = attn.ATTN_DECODE_NOALLOC_SCRATCH_BYTES
    assert re.search(r"ATTN_DECODE_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)32 << 20\)", open(HEADER).read())
    assert attn.attn_decode_workspace_bytes(64, 32, 32, 4096, 128) <= lim
    assert attn.attn_decode_workspace_bytes(128, 32, 8, 8192, 128) <= lim
    assert attn.attn_decode_workspace_bytes(2048, 32, 32, 4096, 128) > lim


def test_decode_noalloc_empty_is_noop(lib):
    assert decode_noalloc(q=NULL, o=NULL, B=0) == 0


def prefill_rope(q=P, k=P, v=P, o=P, B=1, Hq=2, Hkv=2, Sq=8, Skv=8, d=64, causal=1, scale=0.125,
                 lens=NULL, table=P, rows=8, ws=NULL, ws_bytes=0, dtype=attn.ATTN_BF16):
    return attn.attn_prefill_rope_fwd(q, k, v, o, B, Hq, Hkv, Sq, Skv, d, causal, scale, lens, table,
                                      rows, ws, ws_bytes, dtype, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(k=NULL), 1), (dict(table=NULL), 1),
    (dict(rows=7), 2), (dict(rows=0), 2), (dict(Sq=9, Skv=8), 2), (dict(Hq=6, Hkv=4), 2),
    (dict(dtype=attn.ATTN_F32), 3), (dict(d=96), 3),
    (dict(table=MIS), 4), (dict(q=MIS), 4),
    (dict(scale=math.nan), 7),
    (dict(ws=P, ws_bytes=1 * 2 * 8 * 64 * 2 - 1), 5), (dict(ws=MIS, ws_bytes=4096), 4),
])
def test_prefill_rope_rejects(lib, kw, code):
    assert prefill_rope(**kw) == code


def test_prefill_rope_workspace_bytes(lib):
    assert attn.attn_prefill_rope_workspace_bytes(2, 8, 4096, 128) == 2 * 8 * 4096 * 128 * 2
    assert attn.attn_prefill_rope_workspace_bytes(1, 1, 0, 64) == 0
    assert attn.attn_prefill_rope_workspace_bytes(-1, 1, 1, 64) == 0


def prefill_varlen(q=P, k=P, v=P, o=P, cq=P, ck=P, B=2, Hq=4, Hkv=2, mq=64, mk=64, tq=100, tk=100, d=64,
                   causal=1, scale=0.125, dtype=attn.ATTN_BF16):
    return attn.attn_prefill_varlen_fwd(q, k, v, o, cq, ck, B, Hq, Hkv, mq, mk, tq, tk, d, causal,
                                        scale, dtype, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(o=NULL), 1), (dict(k=NULL), 1), (dict(v=NULL), 1),
    (dict(cq=NULL), 1), (dict(ck=NULL), 1),
    (dict(B=-1), 2), (dict(Hq=0), 2), (dict(Hq=6, Hkv=4), 2), (dict(mq=-1), 2), (dict(mk=-1), 2),
    (dict(tq=-1), 2), (dict(tk=-5), 2), (dict(causal=3), 2),
    (dict(mk=(1 << 20), Hkv=16, d=128), 2),                    # one sequence's K rows beyond 2^31 bytes
    (dict(d=96), 3), (dict(dtype=attn.ATTN_F32), 3),
    (dict(q=MIS), 4), (dict(k=MIS), 4), (dict(cq=ctypes.c_void_p(0x10002)), 4),
    (dict(scale=math.inf), 7),
])
def test_prefill_varlen_rejects(lib, kw, code):
    assert prefill_varlen(**kw) == code


def test_prefill_varlen_empty_is_noop(lib):
    assert prefill_varlen(q=NULL, o=NULL, tq=0) == 0
    assert prefill_varlen(q=NULL, o=NULL, mq=0) == 0
    assert prefill_varlen(B=0, cq=NULL, ck=NULL, q=NULL, o=NULL) == 0


def decode_paged(q=P, kp=P, vp=P, o=P, B=2, Hq=4, Hkv=4, d=64, scale=0.125, table=P, max_blocks=4,
                 page=128, pages=8, lens=NULL, dtype=attn.ATTN_BF16, ws=P, wsb=1 << 30):
    return attn.attn_decode_paged_fwd(q, kp, vp, o, B, Hq, Hkv, d, scale, table, max_blocks, page,
                                      pages, lens, dtype, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), 1), (dict(o=NULL), 1), (dict(kp=NULL), 1), (dict(vp=NULL), 1), (dict(table=NULL), 1),
    (dict(page=64), 2), (dict(page=200), 2), (dict(page=0), 2), (dict(max_blocks=0), 2),
    (dict(pages=0), 2), (dict(Hq=6, Hkv=4), 2), (dict(B=-1), 2),
    (dict(max_blocks=1 << 24, page=256), 2),                   # capacity beyond int32
    (dict(max_blocks=(1 << 16) + 1, page=128, d=128), 2),      # one head's rows beyond 2^31 bytes
    (dict(dtype=attn.ATTN_F32, d=96), 3), (dict(dtype=9), 3),
    (dict(d=96), 3), (dict(d=512), 3),
    (dict(q=MIS), 4), (dict(kp=MIS), 4), (dict(table=ctypes.c_void_p(0x10002)), 4), (dict(ws=MIS), 4),
    (dict(ws=NULL), 5), (dict(wsb=16), 5),
    (dict(scale=math.nan), 7),
    (dict(B=65536, Hq=1, Hkv=1), 2),
])
def test_decode_paged_rejects(lib, kw, code):
    assert decode_paged(**kw) == code


def test_decode_paged_empty_batch_is_noop(lib):
    assert decode_paged(B=0, table=NULL, q=NULL, o=NULL) == 0


def test_workspace_bytes(lib):
    ws = attn.attn_decode_workspace_bytes
    assert ws(0, 32, 32, 4096, 128) == 0
    assert ws(1, 6, 4, 64, 128) == 0
    assert ws(1, 32, 32, 4096, 96) == 0
    a = ws(64, 32, 32, 4096, 128)
    assert a > 0 and a % 256 == 0
    # grows with heads and capacity; covers at least one partial per query head
    assert ws(64, 32, 32, 8192, 128) >= a
    assert ws(2, 4, 1, 100, 64) >= 2 * 4 * (64 + 1) * 4


@pytest.mark.parametrize("B,H,S,splits", [
    (64, 32, 4096, 2),     # 2048 heads: two splits (about 4096 workgroups)
    (128, 32, 4096, 1),    # 4096 heads: one
    (16, 32, 8192, 8),     # 512 heads
    (4, 32, 8192, 16),     # 128 heads: capped at 512 keys per split
    (1, 32, 4096, 8),
    (1, 32, 32768, 64),
])
def test_workspace_split_policy(lib, B, H, S, splits):
    """One query head per KV head: the workspace holds exactly the chosen
    splits' partials, B * H * splits rows of d + 1 floats (each part padded
    to 256 bytes); about 4096 workgroups, never below 512 keys per split."""
    rows = B * H * splits
    pad = lambda x: (x + 255) // 256 * 256
    assert attn.attn_decode_workspace_bytes(B, H, H, S, 128) == pad(rows * 128 * 4) + pad(rows * 4)


def test_workspace_head_dim_256(lib):
    """d = 256 decodes: partials of 256 + 1 floats, per split and query head
    on the vector-ALU pass (one query head per KV head), per run and query
    head on the balanced pass (query groups)."""
    ws = attn.attn_decode_workspace_bytes
    # B4 H16: 64 heads -> 8 splits of 512 keys for 4096 keys
    assert ws(4, 16, 16, 4096, 256) >= 4 * 16 * 8 * (256 + 1) * 4
    # B4 H_q16 H_kv8: 4 * 8 heads of 32 units -> 1024 workgroups, (32 + 1024)
    # runs of 2 query heads
    assert ws(4, 16, 8, 4096, 256) >= (4 * 8 + 1024) * 2 * (256 + 1) * 4
    assert ws(1, 32, 32, 4096, 96) == 0


def test_workspace_other_group_sizes(lib, monkeypatch):
    """Group sizes other than 2, 4, 8 and 16 run the balanced pass in column
    blocks of at most 16 query heads (virtual KV heads): a partial per run
    and column of a block, fewer than (virtual heads + workgroups) runs."""
    ws = attn.attn_decode_workspace_bytes
    # B2 H_q28 H_kv4 (groups of 7, one block each): 2 * 4 heads of 32 units
    # -> 256 workgroups, (8 + 256) runs of 7 query heads
    assert ws(2, 28, 4, 4096, 128) >= (8 + 256) * 7 * (128 + 1) * 4
    # B4 H_q32 H_kv1 (one KV head, two blocks of 16): 4 * 2 virtual heads of
    # 16 units -> 128 workgroups, (8 + 128) runs of 16 query heads
    assert ws(4, 32, 1, 2048, 64) >= (8 + 128) * 16 * (64 + 1) * 4
    # the chunk override is for the chunked pass only
    base = ws(1, 3, 1, 1024, 128)
    monkeypatch.setenv("ATTN_DECODE_CHUNK", "256")
    assert ws(1, 3, 1, 1024, 128) == base


def test_workspace_follows_chunk_override(lib, monkeypatch):
    # one query head per KV head: chunked splits
    base = attn.attn_decode_workspace_bytes(1, 4, 4, 4096, 128)
    monkeypatch.setenv("ATTN_DECODE_CHUNK", "256")
    forced = attn.attn_decode_workspace_bytes(1, 4, 4, 4096, 128)
    # 16 splits of 256 keys: 4 heads x 16 x (128 + 1) floats
    assert forced >= 4 * 16 * 129 * 4 and forced >= base


def test_workspace_balanced_query_groups(lib, monkeypatch):
    # query groups use 128-key units spread over at most 1024 workgroups: a
    # partial per run and query head, fewer than B*H_kv + workgroups runs
    # (here 2*2 heads of 8 units: at most 4 + 32 runs of 4 query heads)
    ws = attn.attn_decode_workspace_bytes(2, 8, 2, 1000, 128)
    assert ws >= (2 * 2 + 32) * 4 * 129 * 4
    # the bound does not grow with the cache capacity past 1024 workgroups
    big = attn.attn_decode_workspace_bytes(128, 32, 8, 8192, 128)
    assert big >= (128 * 8 + 1024) * 4 * 129 * 4 and big < 8 << 20
    monkeypatch.setenv("ATTN_DECODE_CHUNK", "4096")     # no effect on the balanced pass
    assert attn.attn_decode_workspace_bytes(2, 8, 2, 1000, 128) == ws


def test_cached_workspace_refused_under_graph_capture(monkeypatch):
    """A graph captured with the cached decode workspace would keep its
    address after a later, larger call regrows (frees) it, so under capture
    the wrapper demands an explicit workspace (checked before any HIP call)."""
    import torch
    import attention_attn_fwd_11_amd as attn
    monkeypatch.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
    with pytest.raises(RuntimeError, match="workspace"):
        attn.workspace_for("cuda:0", 1024)


def test_context_probe_library_exports_and_rejects():
    """libattn_probe.so (measurement context only): every probe entry point
    is exported and invalid arguments return 1 before any HIP call."""
    path = os.path.join(ROOT, "attention_attn_fwd_11_amd", "libattn_probe.so")
    if not os.path.exists(path):
        pytest.skip("libattn_probe.so not built")
    pl = ctypes.CDLL(path)
    for n in ("attn_probe_stream_read", "attn_probe_out_words", "attn_probe_mfma",
              "attn_probe_mfma_operand_bytes", "attn_probe_mfma_flops"):
        assert hasattr(pl, n), n
    pl.attn_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p]
    pl.attn_probe_mfma_operand_bytes.restype = ctypes.c_size_t
    pl.attn_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    pl.attn_probe_mfma_flops.restype = ctypes.c_double
    assert pl.attn_probe_mfma_operand_bytes() == 2 * 4 * 64 * 16
    # blocks x 8 waves x iters x 16 MFMAs x (2 x 32 x 32 x 16) FLOP
    assert pl.attn_probe_mfma_flops(256, 1024) == 256 * 8 * 1024 * 16 * 32768
    assert pl.attn_probe_mfma_flops(0, 5) == 0.0
    assert pl.attn_probe_mfma(NULL, P, 1, 1, NULL) == 1
    assert pl.attn_probe_mfma(P, NULL, 1, 1, NULL) == 1
    assert pl.attn_probe_mfma(MIS, P, 1, 1, NULL) == 1
    assert pl.attn_probe_mfma(P, P, 0, 1, NULL) == 1
    assert pl.attn_probe_mfma(P, P, 1, 0, NULL) == 1
    pl.attn_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p]
    assert pl.attn_probe_stream_read(P, 24, P, 1, NULL) == 1
    assert pl.attn_probe_stream_read(MIS, 32, P, 1, NULL) == 1

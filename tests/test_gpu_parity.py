"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes are compared element by element over the whole output; they
span several tiles and ragged tails in every dimension the kernels tile.
The full-size workloads are compared on sampled rows (each computed by the
oracle one by one) plus properties that hold for every element.
"""
import os
import sys

import numpy as np
import pytest
import torch

import attention_attn_fwd_11_amd as attn
import oracle
from attention_attn_fwd_11_amd import workloads as wl
from tests.gpu_util import assert_close, convex_bound_ok, sample_rows, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(attn.library_path), "libattn.so must be built before GPU tests"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def make(B, Hq, Hkv, Sq, Skv, d, dtype="bf16", seed=0, k_mult=1.0):
    return wl.random_problem(B, Hq, Hkv, Sq, Skv, d, dtype=dtype, device=DEV, seed=seed,
                             k_mult=k_mult)


def lens_tensor(lens):
    return None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)


# ---------------------------------------------------------------------------
# prefill, whole-output comparisons
# ---------------------------------------------------------------------------
PREFILL_CASES = [
    # B, Hq, Hkv, Sq, Skv, d, causal, lens, dtype
    (2, 4, 4, 300, 300, 128, True, None, "bf16"),
    (1, 8, 2, 257, 257, 128, True, None, "bf16"),
    (2, 4, 2, 200, 200, 64, True, None, "bf16"),
    (2, 4, 4, 130, 330, 128, False, None, "bf16"),
    (2, 4, 1, 100, 390, 128, True, None, "bf16"),
    (3, 4, 2, 150, 260, 64, True, [260, 97, 0], "bf16"),
    (2, 2, 2, 64, 64, 128, False, [64, 1], "bf16"),
    (1, 2, 2, 1, 1, 128, True, None, "bf16"),
    # several 256-row tiles with a ragged tail; B*Hkv a multiple of 8 takes
    # the XCD-grouped workgroup order
    (2, 8, 4, 600, 600, 128, True, None, "bf16"),
    (1, 16, 8, 530, 530, 64, True, None, "bf16"),
    (1, 8, 8, 700, 640, 128, False, [640], "bf16"),
    (2, 8, 2, 520, 777, 128, True, [777, 300], "bf16"),
    # d = 256 (four waves, 128-row tiles, 64-key stages)
    (2, 4, 2, 300, 300, 256, True, None, "bf16"),
    (1, 4, 4, 200, 330, 256, False, [330], "bf16"),
    (1, 8, 8, 600, 600, 256, True, None, "bf16"),
    (2, 4, 1, 130, 700, 256, True, [700, 257], "bf16"),
    # causal tile pairs: five tiles (a middle tile alone), four tiles at d = 64
    (1, 4, 2, 1100, 1100, 128, True, None, "bf16"),
    (1, 8, 8, 1024, 1024, 64, True, None, "bf16"),
    (1, 2, 2, 128, 128, 64, True, None, "f32"),
    (2, 4, 2, 200, 260, 128, True, [260, 100], "f32"),
    (1, 3, 1, 70, 90, 64, False, None, "f32"),
    (1, 2, 2, 1, 33, 128, True, [5], "f32"),
    # fp32 key groups: many blocks per group, groups with unequal block
    # counts, an empty sequence; 16-row tiles with a ragged tail at d = 128
    (2, 2, 2, 100, 700, 64, True, [700, 0], "f32"),
    (1, 4, 4, 300, 300, 128, False, None, "f32"),
    # fp32 grids of >= 512 64-row tiles take the 64-row, one-group shape
    (1, 64, 8, 520, 520, 64, True, None, "f32"),
    (1, 64, 16, 512, 600, 128, True, [600], "f32"),
    # fp32 at d = 256: 8-row tiles with key groups (8-key blocks), and the
    # 64-row shape
    (2, 4, 2, 150, 300, 256, True, [300, 41], "f32"),
    (1, 3, 3, 90, 90, 256, False, None, "f32"),
    (1, 64, 64, 520, 520, 256, True, None, "f32"),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=lambda c: "x".join(map(str, c[:6])) + f"-{c[8]}-c{int(c[6])}-l{c[7]}")
def test_prefill_matches_oracle(case):
    B, Hq, Hkv, Sq, Skv, d, causal, lens, dtype = case
    say(f"prefill case {case}")
    x = make(B, Hq, Hkv, Sq, Skv, d, dtype)
    scale = 1.0 / np.sqrt(d)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=causal, scale=scale, kv_lens=lens_tensor(lens))
    torch.cuda.synchronize()
    ref = oracle.attention(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), causal, scale, kv_lens=lens)
    assert_close(o, ref, x["q"].dtype, f"prefill {case}")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_prefill_more_sequences_than_the_ranked_order_covers(d):
    """Above 256 sequences the kernels keep the launch order (no longest-first
    ranking); ragged lengths, empty sequences and both XCD tile maps
    (B * H_kv = 260, not a multiple of 8, and 520, one) must stay exact."""
    g = np.random.default_rng(70 + d)
    for B, Hkv in [(260, 1), (260, 2)]:
        lens = [int(n) for n in g.integers(0, 41, size=B)]
        say(f"prefill B{B} Hkv{Hkv} d{d} ragged lengths, unranked")
        x = make(B, 2 * Hkv, Hkv, 40, 40, d, seed=d + Hkv)
        scale = 1.0 / np.sqrt(d)
        o = attn.prefill(x["q"], x["k"], x["v"], causal=True, scale=scale, kv_lens=lens_tensor(lens))
        torch.cuda.synchronize()
        ref = oracle.attention(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), True, scale, kv_lens=lens)
        assert_close(o, ref, torch.bfloat16, f"prefill B{B} Hkv{Hkv} d{d} unranked")


def test_prefill_workload_f32_small_full():
    w = wl.BY_NAME["prefill_f32_small"]
    say(f"workload {w.name}: {w.describe()}")
    x = wl.generate(w, DEV)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.attention(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), w.causal, w.scale)
    assert_close(o, ref, torch.float32, w.name)


# ---------------------------------------------------------------------------
# decode, whole-output comparisons
# ---------------------------------------------------------------------------
DECODE_CASES = [
    # B, Hq, Hkv, S_cap, d, lens
    (3, 2, 2, 1100, 128, [1100, 1, 0]),
    (3, 4, 2, 1100, 128, [513, 767, 1024]),
    (4, 8, 2, 700, 128, [700, 256, 255, 3]),
    (2, 16, 4, 600, 128, [600, 17]),
    (2, 32, 2, 600, 128, [599, 300]),
    (3, 16, 2, 800, 128, [800, 431, 128]),
    (3, 3, 3, 900, 64, [900, 512, 1]),
    (3, 8, 1, 900, 64, [2, 900, 0]),
    (2, 4, 2, 64, 64, None),
    (3, 8, 2, 1000, 64, [1000, 0, 383]),
    (2, 16, 1, 300, 64, [300, 129]),
    # one split per head (capacity <= 512): the split pass writes O itself
    (4, 2, 2, 500, 128, [500, 1, 0, 257]),
    (2, 3, 3, 512, 64, [512, 77]),
    # other group sizes (3, 5, 7, one KV head for 32 query heads; split and
    # unsplit): column blocks of at most 16 query heads on the matrix cores
    (2, 6, 2, 900, 128, [900, 333]),
    (2, 20, 4, 1300, 128, None),
    (3, 7, 1, 700, 64, [700, 1, 256]),
    (2, 32, 1, 1500, 128, [1500, 1024]),
    (4, 6, 2, 500, 128, [500, 0, 1, 257]),
    # d = 256: one query head per KV head on the vector-ALU pass (split and
    # unsplit); groups of 2, 3, 16 and 20 on the balanced matrix-core pass
    (3, 4, 4, 1100, 256, [1100, 1, 0]),
    (2, 8, 4, 1300, 256, [1300, 200]),
    (2, 6, 2, 500, 256, [500, 17]),
    (3, 16, 1, 700, 256, [700, 0, 129]),
    (2, 40, 2, 400, 256, [31, 400]),
    # groups above 16: blocks of 10 + 10, of 9 + 8, and four blocks of 16
    (2, 40, 2, 800, 64, [800, 129]),
    (2, 17, 1, 600, 128, [600, 300]),
    (1, 64, 1, 1000, 128, None),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "x".join(map(str, c[:5])) + f"-l{c[5]}")
def test_decode_matches_oracle(case):
    B, Hq, Hkv, S, d, lens = case
    say(f"decode case {case}")
    x = make(B, Hq, Hkv, 1, S, d, seed=3)
    scale = 1.0 / np.sqrt(d)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_tensor(lens), scale=scale)
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, scale)
    assert_close(o, ref, torch.bfloat16, f"decode {case}")


@pytest.mark.parametrize("chunk", ["256", "512", "1536"])
def test_decode_split_count_invariance(chunk, monkeypatch):
    """Any split of the cache merges to the same result (within tolerance),
    checked against the oracle for each forced chunk size (one query head per
    KV head: the chunked split pass)."""
    B, Hq, Hkv, S, d = 3, 4, 4, 3000, 128
    lens = [3000, 1537, 255]
    say(f"decode split chunk={chunk}")
    x = make(B, Hq, Hkv, 1, S, d, seed=5, k_mult=4.0)
    monkeypatch.setenv("ATTN_DECODE_CHUNK", chunk)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_tensor(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, 1.0 / np.sqrt(d))
    assert_close(o, ref, torch.bfloat16, f"chunk {chunk}")


BALANCED_PARTITIONS = [(wgs, Hq, 128) for Hq in (8, 6, 40) for wgs in ("1", "3", "7", "64", "100000")]
BALANCED_PARTITIONS += [(wgs, Hq, 256) for Hq in (8, 6) for wgs in ("1", "7", "100000")]


@pytest.mark.parametrize("wgs,Hq,d", BALANCED_PARTITIONS, ids=lambda v: str(v))
def test_decode_balanced_partition_invariance(wgs, Hq, d, monkeypatch):
    """Query groups: the balanced pass spreads 128-key units over a forced
    number of workgroups (one workgroup walking every head, a few, more than
    there are units); every partition merges to the oracle's result.  Lengths
    include 0 and unit boundaries, and batches with no work sit between
    others.  Groups of 4, and of 3 and 20 (column blocks of 3, and 10 + 10
    over two virtual heads per KV head); d = 128 and 256."""
    B, Hkv, S = 9, 2, 1100
    lens = [1100, 0, 128, 129, 0, 255, 256, 1, 0]
    say(f"decode balanced workgroups={wgs} Hq={Hq} d={d}")
    x = make(B, Hq, Hkv, 1, S, d, seed=15, k_mult=4.0)
    monkeypatch.setenv("ATTN_DECODE_WORKGROUPS", wgs)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_tensor(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, 1.0 / np.sqrt(d))
    assert_close(o, ref, torch.bfloat16, f"workgroups {wgs} Hq {Hq} d {d}")


def test_decode_balanced_many_batches():
    """A batch larger than a workgroup's scan width per thread (several
    batches per thread in the prefix sum), ragged lengths with zeros."""
    B, Hq, Hkv, S, d = 300, 4, 1, 300, 64
    g = np.random.default_rng(9)
    lens = [int(x) for x in g.integers(0, S + 1, B)]
    lens[5] = lens[77] = lens[299] = 0
    say("decode balanced B=300")
    x = make(B, Hq, Hkv, 1, S, d, seed=16)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_tensor(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, 1.0 / np.sqrt(d))
    assert_close(o, ref, torch.bfloat16, "B=300")


@pytest.mark.parametrize("d", [128, 256])
def test_decode_balanced_largest_batch(d):
    """The balanced pass at its batch limit (2048 sequences: the unit prefix
    takes 8 batches per thread and 8 KiB of dynamic LDS, beside 128 KiB of
    staging at d = 256), ragged lengths with empty sequences."""
    B, Hq, Hkv, S = 2048, 4, 1, 40
    g = np.random.default_rng(12)
    lens = [int(x) for x in g.integers(0, S + 1, B)]
    lens[0], lens[2047] = S, 0
    say(f"decode balanced B=2048 d={d}")
    x = make(B, Hq, Hkv, 1, S, d, seed=19)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_tensor(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, 1.0 / np.sqrt(d))
    assert_close(o, ref, torch.bfloat16, f"B=2048 d={d}")


MANY_PARTIALS = [
    # Hq, Hkv, forced chunk, forced workgroups, S, lens
    (4, 4, "256", None, 20000, [20000, 8321, 8193, 300, 0]),
    (8, 2, None, "100000", 20000, [20000, 8321, 8193, 300, 0]),
    (6, 2, None, "100000", 20000, [20000, 8321, 8193, 300, 0]),
    # at the four-wave threshold: 64 and 63 partials per head
    (4, 4, "256", None, 16384, [16384, 16128, 16129]),
    (8, 2, None, "100000", 8320, [8192, 8064, 8193]),
]


@pytest.mark.parametrize("Hq,Hkv,chunk,wgs,S,lens", MANY_PARTIALS,
                         ids=["mha-79-splits", "group4-157-runs", "group3-157-runs", "mha-64-63-splits",
                              "group4-64-63-runs"])
def test_decode_merge_of_many_partials(Hq, Hkv, chunk, wgs, S, lens, monkeypatch):
    """Heads with more partials than a wave has lanes (four waves share them,
    each merging 64 at a time with 16 loads in flight): 256-key chunks of a
    20000-key cache (79 splits), and one balanced run per 128-key unit (157
    runs; ragged lengths give 66 and 65; short and empty sequences in the
    same launch take the one-wave merge); and heads with exactly 64 partials
    (four waves) beside 63 (one wave) and 65."""
    B, D = len(lens), 128
    if chunk:
        monkeypatch.setenv("ATTN_DECODE_CHUNK", chunk)
    if wgs:
        monkeypatch.setenv("ATTN_DECODE_WORKGROUPS", wgs)
    say(f"decode many partials Hq={Hq} Hkv={Hkv} chunk={chunk} workgroups={wgs}")
    x = make(B, Hq, Hkv, 1, S, D, seed=18, k_mult=4.0)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_tensor(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, 1.0 / np.sqrt(D))
    assert_close(o, ref, torch.bfloat16, f"many partials Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("Hq,d", [(2, 64), (3, 64), (18, 64), (2, 256), (5, 256)],
                         ids=["group2", "group3", "group18", "group2-d256", "group5-d256"])
def test_decode_chunked_fallback_for_large_batches(Hq, d):
    """Past the balanced pass's batch limit query groups use the chunked
    split pass (groups of 2; of 3, 5 and 18 in column blocks; d = 64 and
    256)."""
    B, Hkv, S = 2100, 1, 40
    g = np.random.default_rng(10)
    lens = [int(x) for x in g.integers(0, S + 1, B)]
    say(f"decode query groups, B=2100 Hq={Hq} d={d} (chunked pass)")
    x = make(B, Hq, Hkv, 1, S, d, seed=17)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=lens_tensor(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), lens, 1.0 / np.sqrt(d))
    assert_close(o, ref, torch.bfloat16, f"B=2100 Hq={Hq} d={d}")


# ---------------------------------------------------------------------------
# invariants the kernels must satisfy exactly
# ---------------------------------------------------------------------------
def test_constant_v_is_returned_exactly():
    say("constant V")
    x = make(2, 4, 2, 200, 200, 128, k_mult=4.0)
    v = x["v"][:, :, :1, :].expand_as(x["v"]).contiguous()
    o = attn.prefill(x["q"], x["k"], v, causal=True)
    exp = v[:, :, :1, :].repeat_interleave(2, dim=1).expand_as(o)
    assert torch.equal(o, exp)
    xd = make(3, 8, 2, 1, 900, 128, seed=9)
    vd = xd["v"][:, :, :1, :].expand_as(xd["v"]).contiguous()
    od = attn.decode(xd["q"], xd["k"], vd, kv_lens=lens_tensor([900, 300, 5]))
    assert torch.equal(od, vd[:, :, :1, :].repeat_interleave(4, dim=1))
    xm = make(2, 4, 4, 1, 700, 128, seed=10)
    vm = xm["v"][:, :, :1, :].expand_as(xm["v"]).contiguous()
    om = attn.decode(xm["q"], xm["k"], vm, kv_lens=lens_tensor([700, 77]))
    assert torch.equal(om, vm[:, :, :1, :])


def test_single_visible_key_returns_its_value():
    say("single key")
    x = make(2, 4, 2, 65, 65, 128, k_mult=8.0)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=True)
    assert torch.equal(o[:, :, 0], x["v"][:, :, 0].repeat_interleave(2, dim=1))
    for G, Hkv in ((1, 4), (4, 2)):
        xd = make(2, G * Hkv, Hkv, 1, 300, 128, seed=11)
        od = attn.decode(xd["q"], xd["k"], xd["v"], kv_lens=lens_tensor([1, 1]))
        assert torch.equal(od[:, :, 0], xd["v"][:, :, 0].repeat_interleave(G, dim=1))


def test_zero_scale_gives_prefix_mean():
    say("zero scale")
    x = make(1, 2, 1, 300, 300, 128)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=True, scale=0.0)
    v = x["v"].double().cpu()[0, 0]
    mean = torch.cumsum(v, 0) / torch.arange(1, 301, dtype=torch.float64)[:, None]
    for h in range(2):
        assert_close(o[0, h], mean.numpy(), torch.bfloat16, "prefix mean")


def test_empty_rows_are_zero():
    say("empty rows")
    x = make(2, 4, 2, 100, 300, 128)
    o = attn.prefill(x["q"], x["k"], x["v"], causal=True, kv_lens=lens_tensor([0, 300]))
    assert torch.count_nonzero(o[0]) == 0
    xd = make(2, 4, 4, 1, 300, 128)
    od = attn.decode(xd["q"], xd["k"], xd["v"], kv_lens=lens_tensor([0, 7]))
    assert torch.count_nonzero(od[0]) == 0 and torch.count_nonzero(od[1]) > 0
    # S_kv = 0: every row empty
    xe = make(1, 2, 2, 5, 1, 64)
    oe = attn.prefill(xe["q"], xe["k"][:, :, :0].contiguous(), xe["v"][:, :, :0].contiguous(),
                      causal=False)
    assert torch.count_nonzero(oe) == 0


def test_gqa_equals_repeated_mha_bitwise():
    say("GQA vs repeated MHA")
    x = make(2, 8, 2, 260, 260, 128, seed=4)
    o1 = attn.prefill(x["q"], x["k"], x["v"], causal=True)
    kr = x["k"].repeat_interleave(4, dim=1).contiguous()
    vr = x["v"].repeat_interleave(4, dim=1).contiguous()
    o2 = attn.prefill(x["q"], kr, vr, causal=True)
    assert torch.equal(o1, o2)


def test_decode_equals_last_prefill_row():
    say("decode vs last prefill row")
    n = 333
    for G in (1, 4):
        x = make(2, 2 * G, 2, n, n, 128, seed=6)
        pre = attn.prefill(x["q"], x["k"], x["v"], causal=True)
        dec = attn.decode(x["q"][:, :, -1:].contiguous(), x["k"], x["v"])
        ref = oracle.decode(x["q"][:, :, -1:].cpu(), x["k"].cpu(), x["v"].cpu(), None,
                            1.0 / np.sqrt(128))
        assert_close(dec, ref, torch.bfloat16, "decode")
        assert_close(dec[:, :, 0], to64(pre[:, :, -1]), torch.bfloat16, "decode vs prefill row")


def test_values_beyond_length_are_never_read():
    """Cache rows at or beyond a sequence's length are filled with NaN; the
    outputs must be bitwise those of a clean cache."""
    say("NaN poison beyond length")
    lens = [1000, 333, 1]
    for Hq, Hkv in ((4, 4), (8, 2)):
        x = make(3, Hq, Hkv, 1, 1100, 128, seed=7)
        lt = lens_tensor(lens)
        clean = attn.decode(x["q"], x["k"], x["v"], kv_lens=lt).clone()
        kp, vp = x["k"].clone(), x["v"].clone()
        for b, n in enumerate(lens):
            kp[b, :, n:] = float("nan")
            vp[b, :, n:] = float("nan")
        poisoned = attn.decode(x["q"], kp, vp, kv_lens=lt)
        assert torch.equal(clean, poisoned)
    xp = make(2, 4, 2, 300, 300, 128, seed=8)
    lt = lens_tensor([300, 123])
    clean = attn.prefill(xp["q"], xp["k"], xp["v"], causal=False, kv_lens=lt).clone()
    kp, vp = xp["k"].clone(), xp["v"].clone()
    kp[1, :, 123:] = float("nan")
    vp[1, :, 123:] = float("nan")
    assert torch.equal(clean, attn.prefill(xp["q"], kp, vp, causal=False, kv_lens=lt))


def test_runs_are_bitwise_deterministic():
    say("determinism")
    x = make(2, 8, 2, 300, 300, 128, seed=12)
    a = attn.prefill(x["q"], x["k"], x["v"], causal=True).clone()
    b = attn.prefill(x["q"], x["k"], x["v"], causal=True)
    assert torch.equal(a, b)
    xd = make(4, 8, 2, 1, 2000, 128, seed=13)
    lt = lens_tensor([2000, 1500, 700, 3])
    a = attn.decode(xd["q"], xd["k"], xd["v"], kv_lens=lt).clone()
    b = attn.decode(xd["q"], xd["k"], xd["v"], kv_lens=lt)
    assert torch.equal(a, b)


def test_side_stream_ordering():
    """Work is enqueued on torch's current stream: results computed on a side
    stream are visible after that stream is synchronised."""
    say("side stream")
    x = make(1, 4, 4, 256, 256, 128, seed=14)
    ref = attn.prefill(x["q"], x["k"], x["v"]).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o = attn.prefill(x["q"], x["k"], x["v"])
    s.synchronize()
    assert torch.equal(o, ref)


# ---------------------------------------------------------------------------
# full-size workloads: sampled rows against the oracle + whole-output checks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["prefill_bf16_b4h32s4096", "prefill_gqa_bf16_h64kv8s16384",
                                  "prefill_bf16_b4h32s4096_d64", "prefill_bf16_b4h16s4096_d256",
                                  "prefill_chunked_gqa_bf16_b16h32kv8q512",
                                  "prefill_noncausal_bf16_b4h32s4096"])
def test_prefill_workload_sampled(name):
    w = wl.BY_NAME[name]
    say(f"workload {name}: {w.describe()}")
    x = wl.generate(w, DEV)
    lens = x["kv_lens"] if w.len_range else None
    o = attn.prefill(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, kv_lens=lens)
    torch.cuda.synchronize()
    ok, finite = convex_bound_ok(o, x["v"], w.Hq)
    assert finite and ok, "output outside the convex hull of V"
    S = w.Sq
    extra = [(0, 0, 0), (w.B - 1, w.Hq - 1, S - 1), (0, w.Hq - 1, 127), (0, 1, 128), (0, 2, S - 129)]
    rows = sample_rows(w.B, w.Hq, S, 250, seed=1, extra=extra)
    ref = oracle.attention_rows(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), w.causal, w.scale, rows,
                                kv_lens=None if lens is None else lens.cpu().tolist())
    idx = torch.tensor(rows, dtype=torch.long)
    got = o[idx[:, 0], idx[:, 1], idx[:, 2]]
    assert_close(got, ref, torch.bfloat16, f"{name} sampled rows")


@pytest.mark.parametrize("name", ["decode_bf16_b64h32l4096", "decode_gqa_bf16_b128h32kv8"])
def test_decode_workload_sampled(name):
    w = wl.BY_NAME[name]
    say(f"workload {name}: {w.describe()}")
    x = wl.generate(w, DEV)
    o = attn.decode(x["q"], x["k"], x["v"], kv_lens=x["kv_lens"], scale=w.scale)
    torch.cuda.synchronize()
    ok, finite = convex_bound_ok(o, x["v"], w.Hq)
    assert finite and ok, "output outside the convex hull of V"
    lens = x["kv_lens"].cpu()
    # a subset of whole batches: shortest, longest and random ones
    order = torch.argsort(lens)
    g = np.random.default_rng(2)
    bsel = sorted({int(order[0]), int(order[-1]), *map(int, g.choice(w.B, 6, replace=False))})
    bt = torch.tensor(bsel, device=DEV)
    q, k, v = x["q"][bt].cpu(), x["k"][bt].cpu(), x["v"][bt].cpu()
    ref = oracle.decode(q, k, v, lens[bsel], w.scale)
    assert_close(o[bt], ref, torch.bfloat16, f"{name} batches {bsel}")

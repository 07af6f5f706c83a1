"""Pins for the CPU oracle: checks of it against facts fixed by the pages and
by mathematics, not against itself.

Each pin_* takes a loaded oracle library handle (so the same pins can be run
against deliberately broken copies of the oracle) and raises AssertionError
when the oracle disagrees.  Sources of each fact:

  - definition of attention, scale then additive mask then softmax then P V:
    "GPU learning day 24: Operator Fusion", section 3.4 (standard attention);
  - the tiled online-softmax loop reaches the same result up to rounding:
    same page, section 3.4 (FlashAttention pseudocode) and FAQ Q1;
  - splitting the KV sequence into parallel parts (Flash-Decoding): same page,
    FAQ Q4; the merge uses the rescaling identity of the section 3.4 loop;
  - decode is attention of one new query over all earlier tokens:
    "Optimizing Decoder Attention for LLMs on GPU", structure of attention in
    decoding mode;
  - closed forms (softmax of equal scores is uniform, one visible key gets
    weight 1, rows of P sum to 1) are properties of softmax itself.
"""
import math

import numpy as np
import torch

import oracle
from oracle import brute, online_model

RNG_SEED = 1234


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def _problem(B, Hq, Hkv, Sq, Skv, d, seed, kscale=1.0):
    q = _rand((B, Hq, Sq, d), seed)
    k = _rand((B, Hkv, Skv, d), seed + 1, kscale)
    v = _rand((B, Hkv, Skv, d), seed + 2)
    return q, k, v


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# Tiny shapes covering every mask / GQA / length combination.
TINY_CASES = [
    # B, Hq, Hkv, Sq, Skv, d, causal, kv_lens
    (1, 1, 1, 1, 1, 1, False, None),
    (1, 2, 2, 3, 3, 4, True, None),
    (2, 4, 2, 3, 5, 3, True, None),
    (2, 4, 1, 4, 4, 2, False, None),
    (2, 4, 4, 2, 6, 3, False, [3, 6]),
    (3, 2, 1, 3, 6, 4, True, [6, 2, 0]),
    (2, 3, 3, 5, 5, 2, True, [5, 3]),
    (1, 4, 2, 1, 7, 5, True, [4]),
]


def pin_brute_force(lib):
    """oracle.c agrees with an independent scalar evaluation on tiny shapes."""
    for n, (B, Hq, Hkv, Sq, Skv, d, causal, lens) in enumerate(TINY_CASES):
        q, k, v = _problem(B, Hq, Hkv, Sq, Skv, d, RNG_SEED + 10 * n)
        scale = 1.0 / math.sqrt(d)
        got = oracle.attention(q, k, v, causal, scale, kv_lens=lens, lib=lib)
        ref = brute.attention(q.tolist(), k.tolist(), v.tolist(), causal, scale, lens)
        _close(got, ref, 1e-13, f"brute case {n}")


def pin_sdpa_library(lib):
    """Special cases that reduce to torch's float64 scaled_dot_product_attention
    (a library routine): square causal, non-causal, GQA, and an explicit
    bottom-right mask for S_q != S_kv."""
    import torch.nn.functional as F
    cases = [(2, 4, 4, 17, 17, 8, True), (1, 6, 2, 9, 9, 16, True),
             (2, 4, 2, 7, 7, 8, False), (1, 2, 1, 5, 12, 8, True), (1, 2, 2, 12, 5, 4, False)]
    for n, (B, Hq, Hkv, Sq, Skv, d, causal) in enumerate(cases):
        q, k, v = _problem(B, Hq, Hkv, Sq, Skv, d, RNG_SEED + 100 + n)
        scale = 0.37
        got = oracle.attention(q, k, v, causal, scale, lib=lib)
        G = Hq // Hkv
        kt = torch.from_numpy(k).repeat_interleave(G, dim=1)
        vt = torch.from_numpy(v).repeat_interleave(G, dim=1)
        mask = None
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Skv)[None, :]
            mask = j <= i + Skv - Sq
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=mask,
                                             scale=scale).numpy()
        _close(got, ref, 1e-12, f"sdpa case {n}")


def pin_online_equals_two_pass(lib):
    """The tiled online-softmax loop equals the two-pass definition for block
    sizes 1, 3, 64, 128 and the whole sequence, with ragged tails."""
    B, Hq, Hkv, S, d = 1, 2, 1, 200, 16
    q, k, v = _problem(B, Hq, Hkv, S, S, d, RNG_SEED + 200, kscale=4.0)
    scale = 1.0 / math.sqrt(d)
    for causal in (True, False):
        ref = oracle.attention(q, k, v, causal, scale, lib=lib)
        for bq, bk in ((1, 1), (3, 3), (64, 64), (128, 64), (64, 128), (S, S), (7, 200)):
            got = online_model.online_attention(q, k, v, causal, scale, block_q=bq, block_k=bk)
            rel = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
            assert rel <= 1e-12, f"online blocks ({bq},{bk}) causal={causal}: rel {rel:.2e}"
    lens = [150]
    ref = oracle.attention(q, k, v, True, scale, kv_lens=lens, lib=lib)
    got = online_model.online_attention(q, k, v, True, scale, kv_lens=lens, block_q=64,
                                        block_k=64)
    _close(got, ref, 1e-12, "online ragged")


def pin_rows_sum_to_one(lib):
    """Each row of P sums to 1 over its visible keys and is 0 on masked keys."""
    B, Hq, Hkv, Sq, Skv, d = 2, 2, 1, 6, 9, 4
    q, k, v = _problem(B, Hq, Hkv, Sq, Skv, d, RNG_SEED + 300)
    lens = [9, 7]
    _, p = oracle.attention(q, k, v, True, 0.5, kv_lens=lens, want_p=True, lib=lib)
    for b in range(B):
        n = lens[b]
        for i in range(Sq):
            vis = np.array([j < n and j <= i + n - Sq for j in range(Skv)])
            row = p[b, :, i, :]
            assert np.all(row[:, ~vis] == 0.0), "masked key with nonzero weight"
            if vis.any():
                assert np.all(row[:, vis] > 0.0), "visible key with zero weight"
                assert np.allclose(row.sum(axis=-1), 1.0, atol=1e-14, rtol=0), "row sum != 1"


def pin_constant_v(lib):
    """If every value row equals the same vector, the output is that vector."""
    B, Hq, Hkv, Sq, Skv, d = 2, 4, 2, 5, 8, 6
    q, k, _ = _problem(B, Hq, Hkv, Sq, Skv, d, RNG_SEED + 400, kscale=3.0)
    c = _rand((B, Hkv, 1, d), RNG_SEED + 401)
    v = np.repeat(c, Skv, axis=2)
    o = oracle.attention(q, k, v, True, 0.3, kv_lens=[8, 6], lib=lib)
    for b in range(B):
        for h in range(Hq):
            _close(o[b, h], np.repeat(c[b, h // 2], Sq, axis=0), 1e-14, "constant V")


def pin_single_key(lib):
    """With one visible key the softmax weight is exactly 1: O = that key's V.
    Covers S_kv = 1, kv_len = 1 and causal row 0 of a square problem."""
    q, k, v = _problem(1, 2, 1, 1, 1, 5, RNG_SEED + 500, kscale=10.0)
    _close(oracle.attention(q, k, v, False, 1.0, lib=lib)[0, :, 0], np.repeat(v[0, 0], 2, axis=0),
           0, "S_kv = 1")
    q, k, v = _problem(2, 2, 2, 1, 6, 5, RNG_SEED + 501, kscale=10.0)
    o = oracle.attention(q, k, v, False, 1.0, kv_lens=[1, 1], lib=lib)
    _close(o[:, :, 0], v[:, :, 0], 0, "kv_len = 1")
    q, k, v = _problem(1, 3, 3, 7, 7, 4, RNG_SEED + 502, kscale=10.0)
    o = oracle.attention(q, k, v, True, 1.0, lib=lib)
    _close(o[0, :, 0], v[0, :, 0], 0, "causal row 0")


def pin_zero_scale_is_prefix_mean(lib):
    """scale = 0 makes every score equal, so each row is the mean of V over its
    visible keys: the causal prefix mean, or the mean of the first kv_len rows."""
    B, Hq, Hkv, S, d = 2, 2, 1, 9, 3
    q, k, v = _problem(B, Hq, Hkv, S, S, d, RNG_SEED + 600, kscale=5.0)
    o = oracle.attention(q, k, v, True, 0.0, lib=lib)
    csum = np.cumsum(v[:, 0], axis=1) / np.arange(1, S + 1)[None, :, None]
    for h in range(Hq):
        _close(o[:, h], csum, 1e-14, "zero-scale causal prefix mean")
    o = oracle.attention(q, k, v, False, 0.0, kv_lens=[4, 9], lib=lib)
    _close(o[0, 0], np.repeat(v[0, 0, :4].mean(axis=0, keepdims=True), S, 0), 1e-14, "len 4 mean")
    _close(o[1, 1], np.repeat(v[1, 0].mean(axis=0, keepdims=True), S, 0), 1e-14, "len 9 mean")


def pin_two_key_closed_form(lib):
    """Hand-derived case: d = 1, q = 1, keys 0 and ln 3, scale 1.  The weights
    are 1/4 and 3/4, so o = (v0 + 3 v1) / 4 and lse = ln 4."""
    q = np.array([[[[1.0]]]])
    k = np.array([[[[0.0], [math.log(3.0)]]]])
    v = np.array([[[[2.0], [-6.0]]]])
    o, lse = oracle.attention(q, k, v, False, 1.0, want_lse=True, lib=lib)
    _close(o.ravel(), [(2.0 + 3 * -6.0) / 4.0], 1e-15, "two-key output")
    _close(lse.ravel(), [math.log(4.0)], 1e-15, "two-key lse")


def pin_large_scores_stable(lib):
    """Scores far beyond exp's range: the max-shifted softmax stays finite and
    puts all weight on the largest score (one-hot limit)."""
    d = 4
    q = np.ones((1, 1, 1, d))
    k = np.zeros((1, 1, 4, d))
    k[0, 0, :, 0] = [1000.0, 3000.0, 2000.0, -5000.0]
    v = _rand((1, 1, 4, d), RNG_SEED + 700)
    o = oracle.attention(q, k, v, False, 1.0, lib=lib)
    _close(o[0, 0, 0], v[0, 0, 1], 1e-15, "one-hot limit")


def pin_gqa_is_repeated_mha(lib):
    """Grouped-query attention equals multi-head attention with each KV head
    repeated over its group of query heads."""
    B, Hq, Hkv, Sq, Skv, d = 2, 6, 2, 4, 7, 5
    q, k, v = _problem(B, Hq, Hkv, Sq, Skv, d, RNG_SEED + 800)
    o = oracle.attention(q, k, v, True, 0.4, kv_lens=[7, 5], lib=lib)
    kr = np.repeat(k, Hq // Hkv, axis=1)
    vr = np.repeat(v, Hq // Hkv, axis=1)
    o2 = oracle.attention(q, kr, vr, True, 0.4, kv_lens=[7, 5], lib=lib)
    _close(o, o2, 1e-15, "GQA vs repeated MHA")


def pin_decode_is_last_causal_row(lib):
    """A decode step (one query over the first n cached keys) equals the last
    row of causal prefill over those n tokens."""
    B, Hq, Hkv, n, d = 2, 4, 2, 11, 6
    q, k, v = _problem(B, Hq, Hkv, n, n, d, RNG_SEED + 900)
    pre = oracle.attention(q, k, v, True, 0.3, lib=lib)
    cap = 16
    kc = np.concatenate([k, _rand((B, Hkv, cap - n, d), 5)], axis=2)
    vc = np.concatenate([v, _rand((B, Hkv, cap - n, d), 6)], axis=2)
    dec = oracle.decode(q[:, :, -1:], kc, vc, [n, n], 0.3, lib=lib)
    _close(dec[:, :, 0], pre[:, :, -1], 1e-14, "decode vs last prefill row")


def pin_key_permutation(lib):
    """Without a causal mask the result does not depend on key order (keys and
    values permuted together)."""
    B, Hq, Hkv, Sq, Skv, d = 1, 2, 1, 3, 10, 4
    q, k, v = _problem(B, Hq, Hkv, Sq, Skv, d, RNG_SEED + 1000)
    perm = np.random.default_rng(3).permutation(Skv)
    o1 = oracle.attention(q, k, v, False, 0.8, lib=lib)
    o2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.8, lib=lib)
    _close(o1, o2, 1e-14, "key permutation")


def pin_split_combine(lib):
    """Split-KV partials merged by log-sum-exp equal the oracle for any
    partition of the keys, including splits that hold no valid key."""
    B, Hq, Hkv, Skv, d = 3, 4, 2, 40, 8
    q, k, v = _problem(B, Hq, Hkv, 1, Skv, d, RNG_SEED + 1100, kscale=4.0)
    lens = [40, 13, 0]
    ref = oracle.decode(q, k, v, lens, 0.35, lib=lib)
    for bounds in ([0], [0, 20], [0, 1, 2, 3, 39], [0, 7, 14, 21, 28, 35], [0, 13, 26]):
        got = online_model.split_combine_attention(q, k, v, lens, 0.35, bounds)
        _close(got, ref, 1e-13, f"split/combine {bounds}")


def pin_empty_rows(lib):
    """A row that sees no key (kv_len = 0, or causal with S_q > kv_len) is 0
    with log-sum-exp -inf."""
    q, k, v = _problem(2, 2, 1, 4, 5, 3, RNG_SEED + 1200)
    o, lse = oracle.attention(q, k, v, True, 1.0, kv_lens=[0, 2], want_lse=True, lib=lib)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0])), "kv_len = 0 row not empty"
    # batch 1: n = 2, S_q = 4: rows 0, 1 see nothing; rows 2, 3 see 1 and 2 keys
    assert np.all(o[1, :, :2] == 0.0) and np.all(np.isneginf(lse[1, :, :2]))
    _close(o[1, :, 2], np.repeat(v[1, 0, 0][None], 2, 0), 0, "first visible row")


def pin_stored_formats(lib):
    """bf16 and fp32 inputs are upcast exactly: the same values stored as
    bf16 bits, fp32 and fp64 give identical results."""
    t = torch.randn(1, 2, 5, 8, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    tk = torch.randn(1, 2, 5, 8, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    tv = torch.randn(1, 2, 5, 8, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    o_bf = oracle.attention(t, tk, tv, True, 0.5, lib=lib)
    o_32 = oracle.attention(t.float(), tk.float(), tv.float(), True, 0.5, lib=lib)
    o_64 = oracle.attention(t.double(), tk.double(), tv.double(), True, 0.5, lib=lib)
    assert np.array_equal(o_bf, o_32) and np.array_equal(o_32, o_64), "stored formats differ"


def pin_rows_entry(lib):
    """The selected-rows entry returns exactly the rows of the full evaluation."""
    B, Hq, Hkv, Sq, Skv, d = 2, 4, 2, 6, 6, 5
    q, k, v = _problem(B, Hq, Hkv, Sq, Skv, d, RNG_SEED + 1300)
    full, lse = oracle.attention(q, k, v, True, 0.6, kv_lens=[6, 4], want_lse=True, lib=lib)
    rows = [(0, 0, 0), (1, 3, 5), (1, 2, 1), (0, 1, 4)]
    got, glse = oracle.attention_rows(q, k, v, True, 0.6, rows, kv_lens=[6, 4], want_lse=True,
                                      lib=lib)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(got[r], full[b, h, i]) and glse[r] == lse[b, h, i]


ALL_PINS = [
    pin_brute_force, pin_sdpa_library, pin_online_equals_two_pass, pin_rows_sum_to_one,
    pin_constant_v, pin_single_key, pin_zero_scale_is_prefix_mean, pin_two_key_closed_form,
    pin_large_scores_stable, pin_gqa_is_repeated_mha, pin_decode_is_last_causal_row,
    pin_key_permutation, pin_split_combine, pin_empty_rows, pin_stored_formats, pin_rows_entry,
]

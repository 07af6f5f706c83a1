"""Workload shapes and seeded synthetic inputs.

This module only describes shapes and draws random numbers; it holds none of
the attention arithmetic, so both the GPU path and the CPU oracle can be fed
from it.

Recipe (the same for every workload), all on one CPU torch.Generator
seeded with `seed`:
  1. if the workload has ragged KV lengths, draw them first: integers
     uniform on [lo, hi], both ends included;
  2. draw Q, then K, then V as float32 standard normals (`torch.randn`);
  3. multiply K by the workload's `k_mult` (a power of two, so exact);
  4. cast to the workload dtype (bf16 by round-to-nearest-even);
  5. copy the result to the target device.
The values do not depend on the device, so the oracle can be evaluated on
the CPU tensors drawn here.
"""
from dataclasses import dataclass, field
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int             # key/value length; for decode, the cache capacity
    d: int
    dtype: str           # "f32" or "bf16"
    causal: bool
    k_mult: float = 1.0
    len_range: tuple = None   # (lo, hi) inclusive for ragged KV lengths
    note: str = field(default="", compare=False)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def describe(self):
        s = (f"{self.kind} {self.dtype} B{self.B} Hq{self.Hq} Hkv{self.Hkv} "
             f"Sq{self.Sq} Skv{self.Skv} d{self.d}")
        if self.causal:
            s += " causal"
        if self.k_mult != 1.0:
            s += f" Kx{self.k_mult:g}"
        if self.len_range:
            s += f" L~U[{self.len_range[0]},{self.len_range[1]}]"
        return s


WORKLOADS = [
    Workload("prefill_f32_small", "prefill", 1, 2, 2, 128, 128, 64, "f32", True,
             note="causal prefill, fp32, oracle-sized"),
    Workload("prefill_bf16_b4h32s4096", "prefill", 4, 32, 32, 4096, 4096, 128, "bf16", True,
             note="causal prefill, bf16 in / fp32 accumulate"),
    Workload("decode_bf16_b64h32l4096", "decode", 64, 32, 32, 1, 4096, 128, "bf16", False,
             note="single-query decode over a bf16 KV cache, every length 4096"),
    Workload("decode_gqa_bf16_b128h32kv8", "decode", 128, 32, 8, 1, 8192, 128, "bf16", False,
             len_range=(256, 8192), note="GQA decode, ragged lengths"),
    Workload("prefill_gqa_bf16_h64kv8s16384", "prefill", 1, 64, 8, 16384, 16384, 128, "bf16",
             True, k_mult=4.0, note="long causal GQA prefill, K scaled by 4"),
    Workload("prefill_bf16_b4h32s4096_d64", "prefill", 4, 32, 32, 4096, 4096, 64, "bf16", True,
             note="causal prefill at head dimension 64"),
    Workload("prefill_bf16_b4h16s4096_d256", "prefill", 4, 16, 16, 4096, 4096, 256, "bf16", True,
             note="causal prefill at head dimension 256 (the headline's FLOPs with half the heads)"),
    Workload("prefill_noncausal_bf16_b4h32s4096", "prefill", 4, 32, 32, 4096, 4096, 128, "bf16",
             False, note="non-causal prefill (every query sees every key)"),
    Workload("prefill_chunked_gqa_bf16_b16h32kv8q512", "prefill", 16, 32, 8, 512, 8192, 128,
             "bf16", True, len_range=(512, 8192),
             note="chunked prefill: 512 new tokens per sequence over a ragged KV cache "
                  "(bottom-right causal)"),
    Workload("decode_gqa_long_bf16_b1h32kv8l131072", "decode", 1, 32, 8, 1, 131072, 128, "bf16",
             False, note="long-context GQA decode: one sequence of 131072 keys"),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def _lengths(w, g):
    if w.len_range is None:
        return torch.full((w.B,), w.Skv, dtype=torch.int32)
    lo, hi = w.len_range
    return torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)


def kv_lengths(w, seed=0):
    """Per-sequence KV lengths (int32, CPU) for workload w: the first draw of
    the recipe."""
    return _lengths(w, torch.Generator(device="cpu").manual_seed(seed))


def generate(w, device="cpu", seed=0):
    """Seeded inputs for workload w, drawn on the CPU and copied to `device`.

    Returns dict(q, k, v, kv_lens) with q [B,Hq,Sq,d], k/v [B,Hkv,Skv,d] in the
    workload dtype and kv_lens int32 [B] (on `device`).
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    lens = _lengths(w, g)
    q = torch.randn((w.B, w.Hq, w.Sq, w.d), generator=g, dtype=torch.float32).to(w.torch_dtype)
    k = torch.randn((w.B, w.Hkv, w.Skv, w.d), generator=g, dtype=torch.float32)
    if w.k_mult != 1.0:
        k.mul_(w.k_mult)
    k = k.to(w.torch_dtype)
    v = torch.randn((w.B, w.Hkv, w.Skv, w.d), generator=g, dtype=torch.float32).to(w.torch_dtype)
    dev = torch.device(device)
    return {"q": q.to(dev), "k": k.to(dev), "v": v.to(dev), "kv_lens": lens.to(dev)}


def random_problem(B, Hq, Hkv, Sq, Skv, d, dtype="bf16", device="cpu", seed=0, k_mult=1.0,
                   len_range=None):
    """Seeded inputs of an arbitrary shape, drawn by the same recipe."""
    w = Workload("adhoc", "prefill", B, Hq, Hkv, Sq, Skv, d, dtype, False, k_mult=k_mult,
                 len_range=len_range)
    return generate(w, device, seed)


def prefill_flops(w, kv_lens=None):
    """Algorithmic FLOPs of one call: 4*d per visible (query, key) pair.

    Two multiply-adds per pair per feature: one for the score, one for P V.
    Masked pairs are not counted.
    """
    lens = kv_lens if kv_lens is not None else torch.full((w.B,), w.Skv)
    i = torch.arange(w.Sq, dtype=torch.int64)
    pairs = 0
    for b in range(w.B):
        n = max(0, min(w.Skv, int(lens[b])))
        if w.causal:
            # query i sees keys j <= i + n - Sq with j < n
            pairs += int((i + (n - w.Sq + 1)).clamp(0, n).sum())
        else:
            pairs += w.Sq * n
    return 4 * w.d * w.Hq * pairs


def decode_kv_bytes(w, kv_lens):
    """Algorithmic K+V bytes of one decode call: every visible cache row of
    every (batch, KV head) read once."""
    elt = 4 if w.dtype == "f32" else 2
    total = sum(max(0, min(w.Skv, int(x))) for x in kv_lens)
    return 2 * total * w.Hkv * w.d * elt


def paged_cache(k, v, kv_lens, page_size, seed=0, spare_pages=3, fill=float("nan")):
    """Lay a contiguous cache k, v [B,Hkv,S,d] out as page pools.

    Each sequence b gets ceil(kv_lens[b] / page_size) pages, drawn in a
    seeded random order from a pool of all needed pages plus `spare_pages`;
    pool rows that hold no valid key (unused pages, rows past a length) are
    set to `fill`, and table entries past a sequence's pages to out-of-range
    values, so a read of either shows up in the output.
    Returns (k_pages, v_pages, block_table) with pools [num_pages,Hkv,P,d]
    and block_table int32 [B, ceil(S / P)] on k's device.
    """
    B, Hkv, S, d = k.shape
    P = page_size
    max_blocks = (S + P - 1) // P
    lens = [max(0, min(S, int(x))) for x in kv_lens]
    need = [(n + P - 1) // P for n in lens]
    num_pages = sum(need) + spare_pages
    g = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(num_pages, generator=g).tolist()
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    kp = torch.full((num_pages, Hkv, P, d), fill, dtype=k.dtype, device=k.device)
    vp = torch.full((num_pages, Hkv, P, d), fill, dtype=v.dtype, device=v.device)
    nxt = 0
    for b in range(B):
        for i in range(max_blocks):
            if i >= need[b]:
                table[b, i] = -7 if i % 2 else num_pages + 1000
                continue
            page = perm[nxt]
            nxt += 1
            table[b, i] = page
            rows = min(P, lens[b] - i * P)
            kp[page, :, :rows] = k[b, :, i * P:i * P + rows]
            vp[page, :, :rows] = v[b, :, i * P:i * P + rows]
    return kp, vp, table.to(k.device)


def varlen_problem(q_lens, k_lens, Hq, Hkv, d, device="cpu", seed=0):
    """Packed sequences by the same recipe (Q, then K, then V as float32
    normals on a CPU generator seeded with `seed`, cast to bf16, copied to
    `device`): q [sum(q_lens), Hq, d], k and v [sum(k_lens), Hkv, d], and the
    int32 offsets cu_q, cu_k [B+1] on `device`."""
    dev = torch.device(device)
    g = torch.Generator(device="cpu").manual_seed(seed)
    tq, tk = int(sum(q_lens)), int(sum(k_lens))
    q = torch.randn((tq, Hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
    k = torch.randn((tk, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
    v = torch.randn((tk, Hkv, d), generator=g, dtype=torch.float32).to(torch.bfloat16).to(dev)
    cu_q = torch.tensor([0] + list(torch.tensor(q_lens).cumsum(0).tolist()), dtype=torch.int32,
                        device=dev)
    cu_k = torch.tensor([0] + list(torch.tensor(k_lens).cumsum(0).tolist()), dtype=torch.int32,
                        device=dev)
    return {"q": q, "k": k, "v": v, "cu_q": cu_q, "cu_k": cu_k}


# Packed variable-length prefill: B sequences, each with as many queries as
# keys, lengths drawn like the ragged decode lengths (seed 0).
VARLEN = Workload("prefill_varlen_gqa_bf16_b16h32kv8", "prefill", 16, 32, 8, 4096, 4096, 128, "bf16",
                  True, len_range=(256, 4096),
                  note="packed causal prefill, lengths U[256, 4096], q and k lengths equal")


def varlen_flops(Hq, d, q_lens, k_lens, causal=True):
    """Algorithmic FLOPs of a packed call: 4*d per visible pair, per sequence
    bottom-right causal."""
    pairs = 0
    for s, n in zip(q_lens, k_lens):
        s, n = int(s), int(n)
        if causal:
            i = torch.arange(s, dtype=torch.int64)
            pairs += int((i + (n - s + 1)).clamp(0, n).sum())
        else:
            pairs += s * n
    return 4 * d * Hq * pairs


def rope_table(rows, d, theta=10000.0, device="cpu"):
    """Rotary-embedding table [rows, d] float32: columns f < d/2 hold
    cos(p * theta^(-2f/d)), columns d/2 + f the matching sin, for positions
    p = 0 .. rows-1 (computed in float64, stored as float32).  An input like
    Q, K and V: both the kernels and the oracle read these values."""
    h = d // 2
    inv = theta ** (-2.0 * torch.arange(h, dtype=torch.float64) / d)
    ang = torch.arange(rows, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cat([ang.cos(), ang.sin()], dim=1).to(torch.float32).to(device)

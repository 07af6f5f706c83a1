"""Benchmark of the fused attention forward on one MI355X.

One step is one pass of the whole hot path on its headline shapes:
  - causal prefill, bf16, B=4, H=32, S=4096, d=128  (the headline workload)
  - single-query decode over a bf16 KV cache, B=64, H=32, L=4096, d=128
    (split-KV pass + log-sum-exp combine).
Inputs are seeded synthetic tensors already resident in device memory when
the timed region starts.  W untimed warm-up steps are followed by K timed
steps between device synchronisations; inside them every kernel call is
bracketed by HIP events on the stream it is launched on.

Printed: one JSON line.  `value` is prefill TFLOP/s (algorithmic FLOPs: 4*d
per visible query/key pair) over the prefill kernel's average event time;
decode KV-read GB/s (algorithmic K+V bytes, every visible row once) is given
beside it, with a roofline object for each against MI355X's published peaks
(dense bf16 MFMA 2516.6 TFLOP/s, HBM 8 TB/s), and the median/min/max of the
per-call times.  The remaining workloads (GQA ragged decode, long GQA
prefill, d = 64 and 256, chunked and packed varlen prefill, paged decode,
RoPE prefill in both key placements, a graph-captured small decode, the
fp32 parity-sized prefill) are timed the same way and reported under
"other_workloads".  The CPU oracle (as it stands) is timed on this host for
every configuration -- whole outputs of the fp32 prefill and both decodes,
a bounded sample of query rows of the two large prefills -- as
"cpu_baseline" (the headline prefill's figure on top, the rest under
"per_config").
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # 256 CUs x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_HBM_GBPS = 8000.0

# Sources that decide what a kernel does: a stored HBM-traffic figure is only
# reported while their hash still matches the one it was measured with.
CSRC = os.path.join(ROOT, "attention_attn_fwd_11_amd", "csrc")
KERNEL_SOURCES = {
    "prefill": ["prefill_bf16.hip", "common.hpp", "kernels.hpp"],
    "decode": ["decode_bf16.hip", "common.hpp", "kernels.hpp", "attn_api.cpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def sources_sha256(kind):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload, kind):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, calibrated against a copy kernel of known size), or None if
    there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["workloads"][workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256") != sources_sha256(kind):
        return None
    return rec["hbm_bytes_per_launch"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (e.g. under a profiler)")
    ap.add_argument("--no-others", action="store_true",
                    help="time only the headline step (prefill + MHA decode)")
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="target CPU time of the oracle sample of each large prefill")
    ap.add_argument("--only", default=None,
                    help="time one named workload only and print its line (for profiling); "
                         "decode_graph_small runs the eager-versus-graph decode comparison")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --only: afterwards run a plain device copy of this many MiB "
                         "(3 times), the reference for calibrating HBM byte counters")
    return ap.parse_args()


class Timer:
    """Accumulates HIP-event time of repeated calls on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __call__(self, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.append((a, b))

    def mean_ms(self):
        ts = [a.elapsed_time(b) for a, b in self.pairs]
        return sum(ts) / len(ts), ts


def spread(ts):
    """Median, min and max of per-call times (ms)."""
    s = sorted(ts)
    n = len(s)
    med = s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])
    return {"median_ms": round(med, 4), "min_ms": round(s[0], 4), "max_ms": round(s[-1], 4)}


def _errors(gpu, ref, dtype):
    """Errors of a GPU result against the oracle's fp64 values, with the bar
    the tests apply: bf16 max-abs <= 2e-2 and mean-abs <= 2e-3; fp32
    norm-wise relative error <= 1e-5."""
    import numpy as np
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    e = np.abs(g - r)
    out = {"elements": int(e.size), "max_abs": float(e.max()) if e.size else 0.0,
           "mean_abs": float(e.mean()) if e.size else 0.0}
    if dtype == "f32":
        out["rel_norm"] = float(np.linalg.norm(g - r) / max(float(np.linalg.norm(r)), 1e-300))
        out["pass"] = out["rel_norm"] <= 1e-5
    else:
        out["pass"] = out["max_abs"] <= 2e-2 and out["mean_abs"] <= 2e-3
    for key in ("max_abs", "mean_abs", "rel_norm"):
        if key in out:
            out[key] = float(f"{out[key]:.3e}")
    return out


def _oracle_rows(w, x, seconds, seed, gpu_o=None):
    """Time the fp64 oracle (oracle.c, as it stands) on a growing sample of
    random (b, h, i) query rows of workload w until about `seconds` of wall
    time.  Returns (algorithmic FLOPs and K+V bytes of the rows done, seconds,
    rows done, errors of the GPU output gpu_o on those rows or None)."""
    import numpy as np
    import oracle

    q, k, v = x["q"], x["k"], x["v"]
    lens = x["kv_lens"].tolist()
    g = np.random.default_rng(seed)
    rows_done, keys, elapsed = 0, 0, 0.0
    refs, gots = [], []
    batch = 16
    while elapsed < seconds:
        rows = np.stack([g.integers(0, w.B, batch), g.integers(0, w.Hq, batch),
                         g.integers(0, w.Sq, batch)], axis=1)
        t0 = time.perf_counter()
        ref = oracle.attention_rows(q, k, v, w.causal, w.scale, rows,
                                    kv_lens=lens if w.len_range else None)
        elapsed += time.perf_counter() - t0
        if gpu_o is not None:
            refs.append(ref)
            gots.append(gpu_o[rows[:, 0], rows[:, 1], rows[:, 2]].numpy())
        for b, _, i in rows.tolist():
            n = min(max(lens[b], 0), w.Skv)
            keys += max(0, min(n, i + n - w.Sq + 1)) if w.causal else n
        rows_done += batch
        batch = min(batch * 2, 4096)
    err = _errors(np.concatenate(gots), np.concatenate(refs), w.dtype) if refs else None
    return 4 * w.d * keys, 2 * 2 * w.d * keys, elapsed, rows_done, err


def cpu_baseline(wl, seconds, inputs=None):
    """The fp64 oracle timed on this host's cores for every configuration, in
    the unit of its GPU figure: TFLOP/s for prefill (algorithmic FLOPs, 4*d
    per visible pair), GB/s for decode (K+V bytes of every visible row).
    The fp32 prefill and the three decodes are evaluated in full; the two large
    prefills on random query rows, about `seconds` each.  The headline
    prefill's entry is the top-level figure.  Where the GPU output of the
    same inputs is at hand (the benchmark's last call), `parity` gives its
    errors against the oracle's values just computed (the tests compare
    every element of every configuration; this is the same check on what
    the benchmark ran)."""
    import oracle

    per = {}
    inputs = inputs or {}

    def host(w):
        # the same tensors the GPU ran on, if they were drawn; else the recipe again
        if w.name in inputs:
            return {key: t.cpu() for key, t in inputs[w.name].items() if key != "o"}
        return wl.generate(w, "cpu")

    def gpu_out(w):
        o = inputs.get(w.name, {}).get("o")
        return None if o is None else o.float().cpu()

    def full(w, reps_seconds=0.5):
        x = host(w)
        lens = x["kv_lens"]
        n, t = 0, 0.0
        while t < reps_seconds or n == 0:
            t0 = time.perf_counter()
            ref = oracle.attention(x["q"], x["k"], x["v"], w.causal, w.scale,
                                   kv_lens=lens if (w.len_range or w.kind == "decode") else None)
            t += time.perf_counter() - t0
            n += 1
        o = gpu_out(w)
        err = None if o is None else _errors(o.numpy(), ref, w.dtype)
        return x, t / n, err

    w1 = wl.BY_NAME["prefill_f32_small"]
    _, t1, e1 = full(w1)
    f1 = wl.prefill_flops(w1)
    per[w1.name] = {"value": f1 / t1 / 1e9, "unit": "GFLOP/s", "seconds_per_call": t1,
                    "sample": "whole output (fp32 inputs)", "parity": e1}
    for name in ("decode_bf16_b64h32l4096", "decode_gqa_bf16_b128h32kv8",
                 "decode_gqa_long_bf16_b1h32kv8l131072"):
        w = wl.BY_NAME[name]
        x, t, err = full(w, 0.0)
        by = wl.decode_kv_bytes(w, x["kv_lens"])
        per[name] = {"value": by / t / 1e9, "unit": "GB/s", "seconds_per_call": t,
                     "sample": "whole output", "parity": err}
    for name in ("prefill_bf16_b4h32s4096", "prefill_gqa_bf16_h64kv8s16384"):
        w = wl.BY_NAME[name]
        x = host(w)
        fl, _, t, rows, err = _oracle_rows(w, x, seconds, seed=0, gpu_o=gpu_out(w))
        full_fl = wl.prefill_flops(w)
        per[name] = {"value": fl / t / 1e12, "unit": "TFLOP/s",
                     "seconds_whole_call_est": full_fl / (fl / t),
                     "sample": f"{rows} random (b, h, i) query rows ({fl / 1e9:.1f} GFLOP fp64, "
                               f"{t:.1f} s)", "parity": err}
    for rec in per.values():
        rec["value"] = round(rec["value"], 6 if rec["unit"] == "TFLOP/s" else 3)
        for key in ("seconds_per_call", "seconds_whole_call_est"):
            if key in rec:
                rec[key] = round(rec[key], 4)
    head = per["prefill_bf16_b4h32s4096"]
    return {
        "value": head["value"],
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "headline prefill: " + head["sample"],
        "per_config": per,
    }


def sustained_clock(torch, fn, seconds=0.3, period=0.005):
    """Graphics clock the GPU holds while `fn` runs back to back: about
    `seconds` of calls are queued, and the driver's current-SCLK line
    (`pp_dpm_sclk`, the entry marked '*') is read every `period` s until they
    finish.  Context only (outside any timed region): the published MFMA
    peak assumes 2.4 GHz.  None when the file is not readable or several
    cards make it ambiguous."""
    import glob
    import re
    files = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
    if len(files) != 1:
        return None

    def read():
        try:
            with open(files[0]) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    if read() is None:
        return None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    per_call = max(time.perf_counter() - t0, 1e-5)
    calls = max(1, int(seconds / per_call))
    for _ in range(calls):
        fn()
    done = torch.cuda.Event()
    done.record()
    time.sleep(0.02)   # let the clock settle under the load
    samples = []
    while not done.query():
        v = read()
        if v is not None:
            samples.append(v)
        time.sleep(period)
    torch.cuda.synchronize()
    if not samples:
        return None
    samples.sort()
    return {"median_mhz": samples[len(samples) // 2], "min_mhz": samples[0], "max_mhz": samples[-1],
            "samples": len(samples)}


def read_probe(torch, dev, gib=4):
    """Rate of a plain streaming-read kernel on this device (the grid-stride
    nontemporal reads of libattn_probe.so over `gib` GiB, best over a few
    launch shapes).  Context only, not a ceiling: the decode kernels, which
    keep more bytes in flight per compute unit, read faster than it.  The
    roofline peak is the published 8 TB/s."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "attention_attn_fwd_11_amd", "libattn_probe.so"))
    lib.attn_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.c_int32, ctypes.c_void_p]
    lib.attn_probe_out_words.argtypes = [ctypes.c_int32]
    lib.attn_probe_out_words.restype = ctypes.c_size_t
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    shapes = [8192, 16384, 32768]
    out = torch.empty(lib.attn_probe_out_words(max(shapes)), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    best = {}
    for blocks in shapes:
        ts = []
        for rep in range(6):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            rc = lib.attn_probe_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, stream)
            b.record()
            if rc != 0:
                raise RuntimeError(f"read probe failed ({rc})")
            torch.cuda.synchronize()
            if rep:
                ts.append(a.elapsed_time(b))
        best[blocks] = nbytes / (min(ts) * 1e-3) / 1e9
    del buf, out
    blocks = max(best, key=best.get)
    return {"gbps": round(best[blocks], 1), "bytes": nbytes, "workgroups": blocks,
            "kernel": "grid-stride 16-byte nontemporal loads, 8 in flight per lane (libattn_probe.so)"}


def mfma_probe(torch, dev, steps, warmup, iters=1024):
    """Rate of back-to-back v_mfma_f32_32x32x16_bf16 from registers
    (libattn_probe.so: two waves per SIMD, one workgroup per compute unit,
    random bf16 operands), timed like the prefill: `warmup` untimed launches,
    then `steps` launches each between HIP events on the current stream, one
    launch lasting about as long as one headline prefill.  Context only: what
    the matrix cores sustain, at the clock the chip holds under that load,
    with no memory, LDS or vector work beside them.  The roofline peak is
    the published 2516.6 TFLOP/s."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "attention_attn_fwd_11_amd", "libattn_probe.so"))
    lib.attn_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_void_p]
    lib.attn_probe_mfma_operand_bytes.restype = ctypes.c_size_t
    lib.attn_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.attn_probe_mfma_flops.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator().manual_seed(7)
    ops = torch.randn(lib.attn_probe_mfma_operand_bytes() // 2, generator=g).to(torch.bfloat16).to(dev)
    out = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.attn_probe_mfma(ops.data_ptr(), out.data_ptr(), cus, iters, stream)
        if rc != 0:
            raise RuntimeError(f"matrix-core probe failed ({rc})")

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(steps):
        tm(launch)
    torch.cuda.synchronize()
    ms, _ = tm.mean_ms()
    flops = lib.attn_probe_mfma_flops(cus, iters)
    res = {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 4), "workgroups": cus,
           "flop_per_launch": flops,
           "kernel": "v_mfma_f32_32x32x16_bf16 only, 4 independent accumulators per wave, 2 waves per SIMD "
                     "(libattn_probe.so)"}
    clk = sustained_clock(torch, launch)
    if clk:
        res["sustained_sclk"] = clk
    del ops, out
    return res


def varlen_prefill(torch, attn, wl, dev, steps, warmup):
    """Packed causal prefill over sequences of mixed lengths (the varlen
    workload: q and k lengths equal, drawn from U[256, 4096])."""
    w = wl.VARLEN
    lens = wl.kv_lengths(w).tolist()
    x = wl.varlen_problem(lens, lens, w.Hq, w.Hkv, w.d, device=dev, seed=0)
    out = torch.empty_like(x["q"])
    f = lambda: attn.prefill_varlen(x["q"], x["k"], x["v"], x["cu_q"], x["cu_k"], max(lens),
                                    max(lens), causal=True, scale=w.scale, out=out)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(steps):
        tm(f)
    torch.cuda.synchronize()
    ms, _ = tm.mean_ms()
    fl = wl.varlen_flops(w.Hq, w.d, lens, lens)
    return {"shape": w.describe() + " packed", "ms": round(ms, 4),
            "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
            "frac_of_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flop": fl, "tokens": sum(lens)}


def rope_prefill(torch, attn, wl, x, w, steps, warmup):
    """The headline causal prefill with the rotary embedding (Q rotated in
    the kernel from a [S, d] fp32 cos/sin table; K rotated per stage in the
    kernel, or once by a pre-pass into a workspace).  The rotation adds no
    MFMA work: the rate counts the same attention FLOPs."""
    table = wl.rope_table(w.Skv, w.d, device=x["q"].device)
    out = torch.empty_like(x["q"])
    ws = torch.empty(attn.attn_prefill_rope_workspace_bytes(w.B, w.Hkv, w.Skv, w.d), dtype=torch.uint8,
                     device=x["q"].device)
    res = {}
    for mode, wsp in (("k_in_kernel", None), ("k_prepass", ws)):
        f = lambda: attn.prefill(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale, out=out,
                                 rope=table, rope_workspace=wsp)
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        tm = Timer(torch)
        for _ in range(steps):
            tm(f)
        torch.cuda.synchronize()
        ms, _ = tm.mean_ms()
        fl = wl.prefill_flops(w)
        res[mode] = {"ms": round(ms, 4), "TFLOP/s": round(fl / (ms * 1e-3) / 1e12, 1),
                     "frac_of_mfma_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return {"shape": w.describe() + " + RoPE", "algorithmic_flop": wl.prefill_flops(w),
            "note": "k_prepass: keys rotated once into a workspace, then Q rotated in the attention "
                    "kernel (ms covers both launches)", **res}


def f32_small(torch, attn, wl, dev, steps, warmup, inputs=None):
    """The fp32 causal prefill B1 H2 S128 d64 (parity-sized; latency-bound, so
    its time is reported without a roofline fraction).  Its tensors and
    output are added to `inputs`."""
    w = wl.BY_NAME["prefill_f32_small"]
    x = wl.generate(w, dev)
    out = torch.empty_like(x["q"])
    if inputs is not None:
        inputs[w.name] = {**x, "o": out}
    f = lambda: attn.prefill(x["q"], x["k"], x["v"], causal=True, scale=w.scale, out=out)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(steps):
        tm(f)
    torch.cuda.synchronize()
    ms, ts = tm.mean_ms()
    return {"shape": w.describe(), "ms": round(ms, 4), **spread(ts),
            "algorithmic_flop": wl.prefill_flops(w)}


def paged_decode(torch, attn, wl, x, w, steps, warmup, page_size=128):
    """The ragged GQA decode with its cache in page_size-key pages (only the
    pages the lengths need, in shuffled order); same algorithmic bytes as the
    contiguous call."""
    lens = x["kv_lens"]
    kp, vp, table = wl.paged_cache(x["k"], x["v"], lens.cpu().tolist(), page_size, seed=8)
    out = torch.empty_like(x["q"])
    f = lambda: attn.decode_paged(x["q"], kp, vp, table, kv_lens=lens, scale=w.scale, out=out)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(steps):
        tm(f)
    torch.cuda.synchronize()
    ms, _ = tm.mean_ms()
    by = wl.decode_kv_bytes(w, lens.cpu())
    del kp, vp
    return {"shape": w.describe() + f" paged P{page_size}", "ms": round(ms, 4),
            "GB/s": round(by / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "algorithmic_bytes": by,
            "pages": sum((int(n) + page_size - 1) // page_size for n in lens.cpu().tolist())}


def decode_graph(torch, attn, wl, dev, steps=192):
    """Launch overhead of a small decode step (B1 H32 L4096 d128, 64 MiB of
    cache): host wall time per step over `steps` back-to-back eager calls,
    against replays of the same call captured in a HIP graph, one step per
    graph and 16 steps per graph; and the host time to issue one eager call
    and one replay (without waiting for the GPU).  A replay costs more host
    time than this step's kernels take, so one-step replays leave the GPU idle
    between steps; capturing several steps per graph amortises that cost."""
    B, H, L, d = 1, 32, 4096, 128
    x = wl.random_problem(B, H, H, 1, L, d, dtype="bf16", device=dev, seed=7)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    out = torch.empty_like(x["q"])
    ws = torch.empty(attn.attn_decode_workspace_bytes(B, H, H, L, d), dtype=torch.uint8, device=dev)
    f = lambda: attn.decode(x["q"], x["k"], x["v"], kv_lens=lens, out=out, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for k in (1, 16):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(k):
                f()
        graphs[k] = g
    torch.cuda.synchronize()

    def wall(fn, calls, per_call):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / (calls * per_call) * 1e6

    def issue(fn, calls=32):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(calls):
            fn()
        t = (time.perf_counter() - t0) / calls * 1e6
        torch.cuda.synchronize()
        return t

    eager_us = wall(f, steps, 1)
    graph_us = wall(graphs[1].replay, steps, 1)
    graph16_us = wall(graphs[16].replay, steps // 16, 16)
    return {"shape": f"decode bf16 B{B} Hq{H} Hkv{H} Sq1 Skv{L} d{d}", "steps": steps,
            "eager_us_per_step": round(eager_us, 2), "graph_us_per_step": round(graph_us, 2),
            "graph16_us_per_step": round(graph16_us, 2),
            "host_us_per_eager_call": round(issue(f), 2),
            "host_us_per_replay": round(issue(graphs[1].replay), 2),
            "kv_bytes": 2 * B * H * L * d * 2}


def only(args, torch, attn, wl, dev):
    """Warm up and time one workload (nothing else launched in between)."""
    w = wl.BY_NAME[args.only]
    x = wl.generate(w, dev)
    o = torch.empty_like(x["q"])
    if w.kind == "prefill":
        lens = x["kv_lens"] if w.len_range else None
        f = lambda: attn.prefill(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale,
                                 kv_lens=lens, out=o)
        work = wl.prefill_flops(w, x["kv_lens"].cpu() if w.len_range else None)
        unit = "TFLOP/s"
    else:
        f = lambda: attn.decode(x["q"], x["k"], x["v"], kv_lens=x["kv_lens"], scale=w.scale, out=o)
        work, unit = wl.decode_kv_bytes(w, x["kv_lens"].cpu()), "GB/s"
    for _ in range(args.warmup):
        f()
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(args.steps):
        tm(f)
    torch.cuda.synchronize()
    ms, all_ms = tm.mean_ms()
    rate = work / (ms * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    peak = PEAK_BF16_TFLOPS if unit == "TFLOP/s" else PEAK_HBM_GBPS
    line = {"workload": w.name, "shape": w.describe(), "ms": round(ms, 4),
            "min_ms": round(min(all_ms), 4), "max_ms": round(max(all_ms), 4),
            "rate": round(rate, 2), "unit": unit, "frac": round(rate / peak, 4),
            "algorithmic_per_launch": work, "steps": args.steps, "warmup": args.warmup,
            "sources_sha256": sources_sha256(w.kind)}
    if args.copy_mib > 0:
        # elementwise x * 1 over bf16: reads and writes copy_mib MiB once each
        n = args.copy_mib * (1 << 20) // 2
        src = torch.randn(n, device=dev).to(torch.bfloat16)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        assert torch.equal(dst, src)
        line["copy_bytes_each_way"] = n * 2
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path: every workload here runs on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch

    import attention_attn_fwd_11_amd as attn
    from attention_attn_fwd_11_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.only == "decode_graph_small":
        print(json.dumps(decode_graph(torch, attn, wl, dev)), flush=True)
        return
    if args.only:
        return only(args, torch, attn, wl, dev)

    wp = wl.BY_NAME["prefill_bf16_b4h32s4096"]
    wd = wl.BY_NAME["decode_bf16_b64h32l4096"]
    others = [] if args.no_others else [wl.BY_NAME[n] for n in (
        "decode_gqa_bf16_b128h32kv8", "prefill_gqa_bf16_h64kv8s16384",
        "prefill_bf16_b4h32s4096_d64", "prefill_bf16_b4h16s4096_d256",
        "prefill_chunked_gqa_bf16_b16h32kv8q512", "prefill_noncausal_bf16_b4h32s4096",
        "decode_gqa_long_bf16_b1h32kv8l131072")]
    inputs = {w.name: wl.generate(w, dev) for w in [wp, wd, *others]}
    torch.cuda.synchronize()

    def call(w):
        x = inputs[w.name]
        if w.kind == "prefill":
            return lambda: attn.prefill(x["q"], x["k"], x["v"], causal=w.causal, scale=w.scale,
                                        kv_lens=x["kv_lens"] if w.len_range else None,
                                        out=x.setdefault("o", torch.empty_like(x["q"])))
        return lambda: attn.decode(x["q"], x["k"], x["v"], kv_lens=x["kv_lens"], scale=w.scale,
                                   out=x.setdefault("o", torch.empty_like(x["q"])))

    fp, fd = call(wp), call(wd)
    for _ in range(args.warmup):
        fp()
        fd()
    torch.cuda.synchronize()

    tp, td = Timer(torch), Timer(torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        tp(fp)
        td(fd)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_p, ts_p = tp.mean_ms()
    ms_d, ts_d = td.mean_ms()

    flops_p = wl.prefill_flops(wp)
    bytes_d = wl.decode_kv_bytes(wd, inputs[wd.name]["kv_lens"].cpu())
    tflops = flops_p / (ms_p * 1e-3) / 1e12
    gbps = bytes_d / (ms_d * 1e-3) / 1e9

    other = {}
    for w in others:
        f = call(w)
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        tm = Timer(torch)
        for _ in range(args.steps):
            tm(f)
        torch.cuda.synchronize()
        ms, _ = tm.mean_ms()
        if w.kind == "prefill":
            fl = wl.prefill_flops(w, inputs[w.name]["kv_lens"].cpu() if w.len_range else None)
            rate = fl / (ms * 1e-3) / 1e12
            other[w.name] = {"shape": w.describe(), "ms": round(ms, 4), "TFLOP/s": round(rate, 1),
                             "frac_of_mfma_peak": round(rate / PEAK_BF16_TFLOPS, 4),
                             "algorithmic_flop": fl}
        else:
            by = wl.decode_kv_bytes(w, inputs[w.name]["kv_lens"].cpu())
            rate = by / (ms * 1e-3) / 1e9
            other[w.name] = {"shape": w.describe(), "ms": round(ms, 4), "GB/s": round(rate, 1),
                             "frac_of_hbm_peak": round(rate / PEAK_HBM_GBPS, 4),
                             "algorithmic_bytes": by}

    roof_p = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
              "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
              "traffic": measured_traffic(wp.name, "prefill"), "traffic_unit": "bytes/launch",
              "kernel": "prefill_bf16_kernel<128, true, 0>", "avg_launch_ms": round(ms_p, 4),
              "algorithmic_per_launch": flops_p}
    roof_d = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": round(gbps / PEAK_HBM_GBPS, 4),
              "traffic": measured_traffic(wd.name, "decode"), "traffic_unit": "bytes/launch",
              "kernel": "decode_split_valu<128> + decode_combine<128, 1>",
              "avg_launch_ms": round(ms_d, 4), "algorithmic_per_launch": bytes_d}
    dominant, second = (roof_p, roof_d) if ms_p >= ms_d else (roof_d, roof_p)

    out = {
        "metric": "prefill attention TFLOPS + decode KV GB/s, % of MI355X peak (1 GPU)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), drawn on the host by the documented recipe, "
                "copied to the device before timing)",
        "config": {
            "workload": "causal prefill bf16 B4 H32 S4096 d128 + decode bf16 B64 H32 L4096 d128",
            "prefill": wp.describe(), "decode": wd.describe(),
            "prefill_ms": round(ms_p, 4), "decode_ms": round(ms_d, 4),
            "prefill_spread": spread(ts_p), "decode_spread": spread(ts_d),
        },
        "prefill_tflops": round(tflops, 2),
        "prefill_frac_of_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "decode_kv_gbps": round(gbps, 1),
        "decode_frac_of_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "roofline": dominant,
        "roofline_other": second,
        "other_workloads": other,
    }
    if not args.no_others:
        wg = wl.BY_NAME["decode_gqa_bf16_b128h32kv8"]
        other["decode_paged_gqa_bf16_b128h32kv8_p128"] = paged_decode(
            torch, attn, wl, inputs[wg.name], wg, args.steps, args.warmup)
        other[wl.VARLEN.name] = varlen_prefill(torch, attn, wl, dev, args.steps, args.warmup)
        other["prefill_rope_bf16_b4h32s4096"] = rope_prefill(torch, attn, wl, inputs[wp.name], wp,
                                                             args.steps, args.warmup)
    other["decode_graph_small"] = decode_graph(torch, attn, wl, dev)
    other["prefill_f32_small"] = f32_small(torch, attn, wl, dev, args.steps, args.warmup, inputs)
    probe = read_probe(torch, dev)
    out["context"] = {
        "streaming_read_probe": probe,
        "note": "a simple streaming-read kernel's rate, for context; not a ceiling (the decode "
                "kernels exceed it)",
        "decode_over_probe": round(gbps / probe["gbps"], 4),
    }
    props = torch.cuda.get_device_properties(dev)
    out["context"]["device"] = {
        "name": props.name, "arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "memory_gib": round(props.total_memory / 2**30, 1),
        "hip": getattr(torch.version, "hip", None), "torch": torch.__version__}
    mp = mfma_probe(torch, dev, args.steps, args.warmup)
    out["context"]["mfma_probe"] = mp
    out["context"]["prefill_frac_of_mfma_probe"] = round(tflops / mp["tflops"], 4)
    clk_p, clk_d = sustained_clock(torch, fp), sustained_clock(torch, fd)
    if clk_p or clk_d:
        out["context"]["sustained_sclk"] = {
            "prefill": clk_p, "decode": clk_d,
            "source": "pp_dpm_sclk sampled while each headline workload ran back to back, after the "
                      "timed steps; the published MFMA peak assumes 2400 MHz"}
        if clk_p:
            out["context"]["prefill_frac_of_peak_at_sustained_clock"] = round(
                tflops / (PEAK_BF16_TFLOPS * clk_p["median_mhz"] / 2400.0), 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Build libattn.so (the gfx950 kernels and the C ABI), libattn_probe.so
(the streaming-read and matrix-core probes the benchmark uses for context) and
libattn_lds_poison.so (the same library with every direct global -> LDS copy
preceded by a NaN fill of its destination, a debug build the tests use to
catch missing waits and barriers), with hipcc.

    python -m attention_attn_fwd_11_amd.build

Objects go to _build/ at the repository root; the library lands next to this
file.  Every source is compiled for gfx950 only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
PROBE_LIB = os.path.join(PKG, "libattn_probe.so")
POISON_LIB = os.path.join(PKG, "libattn_lds_poison.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["attn_api.cpp", "prefill_f32.hip", "prefill_bf16.hip", "prefill_d256.hip", "decode_bf16.hip",
           "decode_f32.hip", "util.hip", "rope_bf16.hip"]
PROBE_SOURCES = ["read_probe.hip"]
# Sources that stage tiles in LDS by direct copies: rebuilt with
# ATTN_LDS_POISON for the poison library (the rest is shared).
POISON_SOURCES = ["prefill_bf16.hip", "prefill_d256.hip", "decode_bf16.hip"]

# Device code for gfx950 only.  Packed-fp32 instruction selection is switched
# off on purpose: ordinary fp32 code is compiled to scalar-lane VALU ops.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-I", os.path.join(ROOT, "include"),
]


# Per-source device flags.  The prefill kernels at d = 256 need more than
# 256 registers per lane; by default the compiler puts the MFMA output
# accumulator in the accumulation registers and copies it into vector
# registers on every K/V stage (for the rare rescale of the accumulator).
# MFMA results in vector registers leave the accumulation registers to
# values the matrix cores only read, with no copies and no spills.
SOURCE_FLAGS = {
    "prefill_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "prefill_d256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src, extra, suffix=""):
    out = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    # keep real warnings visible; drop the host pass's note about the gfx feature flag
    warn = [l for l in (r.stderr or "").splitlines()
            if l.strip() and "packed-fp32-ops" not in l and "not a recognized feature" not in l]
    return out, "\n".join(warn)


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)


def build(extra=(), verbose=False):
    """Compile every source, link libattn.so, libattn_probe.so and
    libattn_lds_poison.so; returns the path of libattn.so."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, list(extra), "") for src in SOURCES + PROBE_SOURCES]
    jobs += [(src, [*extra, "-DATTN_LDS_POISON"], "_lds_poison") for src in POISON_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        outs = list(ex.map(lambda j: _compile(*j), jobs))
    results = {(src, suffix): out for (src, _, suffix), out in zip(jobs, outs)}
    for obj, warn in outs:
        if warn and verbose:
            print(warn, file=sys.stderr)
    _link([results[(s, "")][0] for s in SOURCES], LIB)
    _link([results[(s, "")][0] for s in PROBE_SOURCES], PROBE_LIB)
    _link([results[(s, "_lds_poison" if s in POISON_SOURCES else "")][0] for s in SOURCES], POISON_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""oracle.c built with AddressSanitizer and UndefinedBehaviorSanitizer, run
over every pin and the mixed-format and rows entries (CPU only).

The oracle is loaded into Python through ctypes, so the sanitizer runtimes
are preloaded into a child interpreter; any report (out-of-bounds access,
use after free, signed overflow, misaligned load, ...) aborts the child and
fails the test.  Leak checking is off: the interpreter itself keeps memory
until exit.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]

CHILD = r"""
import sys
import numpy as np
import oracle
from tests import oracle_pins
lib = oracle.load(sys.argv[1])
for pin in oracle_pins.ALL_PINS:
    pin(lib)
    print("ok", pin.__name__, flush=True)
# rows entry on ragged lengths, selected rows at the edges, bf16 storage
import torch
g = torch.Generator().manual_seed(3)
q = torch.randn(2, 4, 37, 64, generator=g).to(torch.bfloat16)
k = torch.randn(2, 2, 53, 64, generator=g).to(torch.bfloat16)
v = torch.randn(2, 2, 53, 64, generator=g).to(torch.bfloat16)
full = oracle.attention(q, k, v, True, 0.125, kv_lens=[53, 0], lib=lib)
rows = [(0, 0, 0), (0, 3, 36), (1, 1, 5), (1, 3, 36)]
got = oracle.attention_rows(q, k, v, True, 0.125, rows, kv_lens=[53, 0], lib=lib)
assert all(np.array_equal(got[r], full[b, h, i]) for r, (b, h, i) in enumerate(rows))
print("SANITIZED_OK", flush=True)
"""


def _runtime(name):
    cc = os.environ.get("CC", "gcc")
    try:
        path = subprocess.run([cc, f"-print-file-name={name}"], capture_output=True, text=True,
                              check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("the C compiler ships no sanitizer runtimes")
    lib = oracle_build.build(str(tmp_path / "liboracle_san.so"), extra=SAN, quiet=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", CHILD, lib], capture_output=True, text=True,
                       cwd=ROOT, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "SANITIZED_OK" in r.stdout, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]

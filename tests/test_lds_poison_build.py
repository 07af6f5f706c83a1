"""The LDS-poison debug build really poisons (CPU only: compiles to gfx950
assembly, runs nothing).

With ATTN_LDS_POISON every direct global -> LDS copy (global_load_lds_dwordx4,
buffer_load_dwordx4 ... lds) must be preceded by the NaN fill of its
destination (ds_write_b128 of 0x7fc17fc1 words) and a wait for LDS writes, so
the copy's data, not the fill, is what a correctly ordered read sees.  The
normal build must contain none of it.  Checked on the balanced decode and the
d = 256 prefill (the bf16 prefill shares the copy helpers).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_attn_fwd_11_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COPY = re.compile(r"(global_load_lds_dwordx4|buffer_load_dwordx4\b.*\blds\b)")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "--cuda-device-only", "-S"]


def asm(src, tmp_path, poison):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + (".poison.s" if poison else ".s"))
    extra = ["-mllvm", "-amdgpu-mfma-vgpr-form"] if src.startswith("prefill") else []
    cmd = [HIPCC, *FLAGS, *extra, *(["-DATTN_LDS_POISON"] if poison else []),
           os.path.join(CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().split("\n")


@pytest.mark.parametrize("src", ["decode_bf16.hip", "prefill_d256.hip"])
def test_poison_build_fills_before_every_copy(src, tmp_path):
    normal, poison = asm(src, tmp_path, False), asm(src, tmp_path, True)
    fill = "0x7fc17fc1"
    assert not any(fill in l for l in normal), "the normal build must not poison"
    assert any(fill in l for l in poison)
    copies = [i for i, l in enumerate(poison) if COPY.search(l)]
    assert len(copies) == sum(1 for l in normal if COPY.search(l)) > 0
    for i in copies:
        # the nearest preceding wait (within the copy's address set-up) is
        # the fill's wait for LDS writes
        window = poison[max(0, i - 12):i]
        assert any("s_waitcnt lgkmcnt(0)" in l for l in window), f"copy at line {i} issued without the fill's wait"
    # one fill per copy site; the compiler may hoist the fill shared by the
    # two paths (whole rows, clamped rows) of a copy into their common block
    writes_p = sum(1 for l in poison if "ds_write_b128" in l)
    writes_n = sum(1 for l in normal if "ds_write_b128" in l)
    assert writes_p - writes_n >= 0.9 * len(copies), (writes_p, writes_n, len(copies))

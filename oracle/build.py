"""Build the oracle's shared library (test infrastructure only).

Compiles oracle.c with the host C compiler and OpenMP into liboracle.so next
to this file.  Nothing here touches the GPU or the product library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
OUT = os.path.join(HERE, "liboracle.so")


def build(out=OUT, src=SRC, extra=(), quiet=False):
    """Compile `src` into the shared library `out`; returns `out`."""
    cc = os.environ.get("CC", "gcc")
    cmd = [cc, "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-Wall", "-Wextra",
           *extra, src, "-o", out + ".tmp", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    os.replace(out + ".tmp", out)
    if not quiet:
        print("built", out)
    return out


if __name__ == "__main__":
    build(*sys.argv[1:2])

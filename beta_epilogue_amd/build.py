"""Build step for the HIP library: one hipcc line, gfx950 only, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgemm_epi.so")
SOURCES = [os.path.join(HERE, "csrc", "gemm_epi.hip")]
HEADERS = [os.path.join(HERE, "csrc", "gemm_epi_kernel.hpp"),
           os.path.join(ROOT, "include", "gemm_epi.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep packed-fp32 instructions out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-pass-failed", "-Wno-inline-asm",
]


def hipcc_command(out: str, extra=()):
    return (["hipcc"] + HIPCC_FLAGS + list(extra) +
            ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
             "-o", out] + SOURCES)


def build(verbose: bool = False, extra=()) -> str:
    """Compile libgemm_epi.so next to this file (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp, extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if "packed-fp32-ops" not in ln and ln.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

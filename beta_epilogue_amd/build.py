"""Build step for the HIP libraries: hipcc, gfx950 only, in-tree.

libgemm_epi.so is linked from gemm_epi.hip (C ABI, variant table) and
GEMM_EPI_PARTS objects of gemm_epi_part.hip, each compiling the kernel
variants of gemm_epi_variants.inc assigned to it; the parts compile in
parallel.  libmfma_ceiling.so is a measurement tool for bench.py.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgemm_epi.so")
MAIN_SOURCE = os.path.join(CSRC, "gemm_epi.hip")
SPLITK_SOURCE = os.path.join(CSRC, "gemm_epi_splitk.hip")
PREP_SOURCE = os.path.join(CSRC, "gemm_epi_prep.hip")
PART_SOURCE = os.path.join(CSRC, "gemm_epi_part.hip")
GEMM_EPI_PARTS = 16
SOURCES = [MAIN_SOURCE, PART_SOURCE, SPLITK_SOURCE, PREP_SOURCE]
HEADERS = [os.path.join(CSRC, "gemm_epi_kernel.hpp"), os.path.join(CSRC, "gemm_epi_launch.hpp"),
           os.path.join(CSRC, "gemm_epi_splitk.hpp"), os.path.join(CSRC, "gemm_epi_prep.hpp"),
           os.path.join(CSRC, "gemm_epi_raster.hpp"), os.path.join(CSRC, "gemm_epi_variants.inc"),
           os.path.join(ROOT, "include", "gemm_epi.h")]
# measurement tool used by bench.py --mfma-ceiling (not part of the GEMM path)
CEILING_LIB = os.path.join(HERE, "libmfma_ceiling.so")
CEILING_SOURCE = os.path.join(CSRC, "mfma_ceiling.hip")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep packed-fp32 instructions out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-pass-failed", "-Wno-inline-asm",
]
INCLUDES = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if "packed-fp32-ops" not in ln and ln.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(cmd), err))
    if verbose and err:
        print(err, file=sys.stderr)


def _jobs() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("MAX_JOBS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def _variant_subset(tmp: str, names) -> list:
    """A copy of the variant table holding only the named variants, in an
    include directory searched before csrc/ (a partial build for
    development; the library then has only those kernels)."""
    src = os.path.join(CSRC, "gemm_epi_variants.inc")
    keep, found = [], set()
    for line in open(src):
        if line.startswith("X("):
            name = line.rsplit('"', 2)[1]
            if name not in names:
                continue
            found.add(name)
        keep.append(line)
    missing = set(names) - found
    if missing:
        raise ValueError("unknown variants: %s" % ", ".join(sorted(missing)))
    d = os.path.join(tmp, "subset")
    os.makedirs(d)
    with open(os.path.join(d, "gemm_epi_variants.inc"), "w") as f:
        f.writelines(keep)
    return ["-I", d]


def build(verbose: bool = False, extra=(), only=None, cache_dir=None) -> str:
    """Compile libgemm_epi.so and libmfma_ceiling.so next to this file.
    Recompiles everything, unless cache_dir names a directory of objects from
    an earlier build with the same options: then an object newer than its
    source and every header is reused (a development shortcut).  only:
    variant names to compile (default: every variant; the GEMM_EPI_ONLY
    environment variable, comma-separated, sets it too)."""
    extra = list(extra)
    if only is None and os.environ.get("GEMM_EPI_ONLY"):
        only = [n for n in os.environ["GEMM_EPI_ONLY"].split(",") if n]
    with tempfile.TemporaryDirectory(prefix="gemm_epi_build_") as tmp:
        if only:
            extra = extra + _variant_subset(tmp, set(only))
        objdir = cache_dir or tmp
        os.makedirs(objdir, exist_ok=True)
        kernel_deps = [os.path.join(CSRC, f) for f in ("gemm_epi_kernel.hpp", "gemm_epi_launch.hpp",
                                                        "gemm_epi_raster.hpp", "gemm_epi_variants.inc")]

        def obj(name, source, deps, defines=()):
            out = os.path.join(objdir, name)
            newest = max(os.path.getmtime(f) for f in [source] + deps)
            if cache_dir and not only and os.path.exists(out) and os.path.getmtime(out) > newest:
                return out, None
            return out, ["hipcc"] + HIPCC_FLAGS + extra + INCLUDES + list(defines) + ["-c", "-o", out, source]

        units = [obj("part%d.o" % k, PART_SOURCE, kernel_deps, ["-DGEMM_EPI_PART=%d" % k])
                 for k in range(GEMM_EPI_PARTS)]
        units += [obj("main.o", MAIN_SOURCE, HEADERS),
                  obj("splitk.o", SPLITK_SOURCE, [os.path.join(CSRC, "gemm_epi_splitk.hpp"),
                                                  os.path.join(CSRC, "gemm_epi_raster.hpp")]),
                  obj("prep.o", PREP_SOURCE, [os.path.join(CSRC, "gemm_epi_prep.hpp")])]
        jobs = [cmd for _, cmd in units if cmd]
        ceil_tmp = CEILING_LIB + ".tmp%d" % os.getpid()
        jobs.append(["hipcc"] + HIPCC_FLAGS + INCLUDES + ["-shared", "-o", ceil_tmp, CEILING_SOURCE])
        with ThreadPoolExecutor(max_workers=_jobs()) as ex:
            for f in [ex.submit(_run, c, verbose) for c in jobs]:
                f.result()
        lib_tmp = LIB + ".tmp%d" % os.getpid()
        _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib_tmp] + [o for o, _ in units],
             verbose)
        os.replace(ceil_tmp, CEILING_LIB)
        os.replace(lib_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""CPU oracle for the fused-epilogue batched GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  The GPU library never loads it and shares no code with it.

The arithmetic lives in ``gemm_epi_oracle.c`` (plain C, fp64, one output
element at a time, k ascending); this module builds it with gcc on first use
and marshals numpy buffers through ctypes.  It computes, per the CuTe DSL
example ``custom_epilogue_dense_gemm.py`` (module docstring, "Tensor
dimensions", and its fused epilogue):

    Y = A . B^T (per batch)      D = alpha*Y + beta*C + x_factor*X

or, with ``relu=True`` (the form the example's epilogue function builds),
D = max(0, alpha*Y + beta*C) + x_factor*X, returning double-precision D, Y and the side sum S = sum_k |a||b| that the
normalised error bound divides by.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gemm_epi_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

# The oracle's own type numbering (see the enum in gemm_epi_oracle.c).
TYPES = {"none": 0, "f16": 1, "bf16": 2, "e4m3": 3, "i8": 4, "f32": 5, "i32": 6,
         "e5m2": 7, "u8": 8}
# numpy container for the raw stored bits of each type
STORAGE = {"f16": np.uint16, "bf16": np.uint16, "e4m3": np.uint8, "e5m2": np.uint8,
           "i8": np.int8, "u8": np.uint8, "f32": np.float32, "i32": np.int32}


class _Desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("L", ctypes.c_int64),
                ("a_mmajor", ctypes.c_int32), ("b_nmajor", ctypes.c_int32),
                ("cd_mmajor", ctypes.c_int32), ("ab_type", ctypes.c_int32),
                ("c_type", ctypes.c_int32), ("x_type", ctypes.c_int32),
                ("b_type", ctypes.c_int32)]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    with _lock:
        if force or not os.path.exists(_LIB) or \
                os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            tmp = _LIB + ".tmp%d" % os.getpid()
            compile_to(tmp)
            os.replace(tmp, _LIB)
    return _LIB


class Oracle:
    """ctypes front end of one oracle shared library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        lib.orc_decode.argtypes = [ctypes.c_int, P, ctypes.c_int64, P]
        lib.orc_gemm_epi_full.argtypes = [ctypes.POINTER(_Desc), P, P, P, P,
                                          ctypes.c_double, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_int, P, P, P,
                                          ctypes.c_int]
        lib.orc_gemm_epi_points.argtypes = [ctypes.POINTER(_Desc), P, P, P, P,
                                            ctypes.c_double, ctypes.c_double,
                                            ctypes.c_double, ctypes.c_int,
                                            ctypes.c_int64, P, P, P, P, ctypes.c_int]
        self.lib = lib
        self.path = lib_path

    def decode(self, type_name, stored):
        return _decode(self.lib, type_name, stored)

    def gemm_epi(self, *a, **kw):
        return _gemm_epi(self.lib, *a, **kw)

    def gemm_epi_points(self, *a, **kw):
        return _gemm_epi_points(self.lib, *a, **kw)


def compile_to(path: str, source: str = None) -> str:
    """Compile ``source`` (default: the oracle's own C text) into ``path``."""
    src_file = _SRC
    tmp_src = None
    if source is not None:
        tmp_src = path + ".c"
        with open(tmp_src, "w") as f:
            f.write(source)
        src_file = tmp_src
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-ffp-contract=off", "-fno-fast-math", "-o", path,
                    src_file, "-lm"], check=True)
    return path


def default() -> Oracle:
    global _lib
    if _lib is None:
        build(force=False)
        _lib = Oracle(_LIB)
    return _lib


def _load():
    return default().lib


def host_threads() -> int:
    """Threads the oracle uses: every core this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _bits(arr, type_name):
    """Raw stored elements as a C-contiguous numpy array of the storage type."""
    if arr is None:
        return None
    if hasattr(arr, "detach"):  # a torch CPU tensor
        import torch
        t = arr.detach().contiguous()
        if t.device.type != "cpu":
            raise ValueError("oracle inputs must be host tensors")
        view = {"f16": torch.int16, "bf16": torch.int16, "e4m3": torch.uint8, "e5m2": torch.uint8,
                "i8": torch.int8, "u8": torch.uint8, "f32": torch.float32, "i32": torch.int32}
        arr = t.view(view[type_name]).numpy()
    a = np.ascontiguousarray(arr).view(STORAGE[type_name])
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _decode(lib, type_name: str, stored) -> np.ndarray:
    a = _bits(stored, type_name).reshape(-1)
    out = np.empty(a.size, dtype=np.float64)
    rc = lib.orc_decode(TYPES[type_name], _ptr(a), a.size, _ptr(out))
    if rc:
        raise ValueError("orc_decode failed (%d)" % rc)
    return out


def _desc(M, N, K, L, a_major, b_major, cd_major, ab, c, x, b=None):
    if a_major not in "KM" or b_major not in "KN" or cd_major not in "NM":
        raise ValueError("bad majorness")
    return _Desc(M, N, K, L, int(a_major == "M"), int(b_major == "N"),
                 int(cd_major == "M"), TYPES[ab], TYPES[c or "none"],
                 TYPES[x or "none"], TYPES[b] if b and b != ab else 0)


def _gemm_epi(lib, M, N, K, L, A, B, C=None, X=None, *, ab="f16", b=None, c=None, x=None,
             a_major="K", b_major="K", cd_major="N", alpha=1.0, beta=0.0,
             x_factor=0.0, relu=False, nthreads=None):
    """Full oracle result: (D_ref, Y_ref, S) as flat float64 arrays laid out
    like C/D (packed batches, L outermost, ``cd_major`` contiguous).  relu:
    D = max(0, alpha*Y + beta*C) + x_factor*X."""
    d = _desc(M, N, K, L, a_major, b_major, cd_major, ab, c, x, b)
    a, b = _bits(A, ab), _bits(B, b or ab)
    cc = _bits(C, c) if c else None
    xx = _bits(X, x) if x else None
    _check_sizes(M, N, K, L, a, b, cc, xx)
    n = M * N * L
    D = np.empty(n, np.float64)
    Y = np.empty(n, np.float64)
    S = np.empty(n, np.float64)
    rc = lib.orc_gemm_epi_full(ctypes.byref(d), _ptr(a), _ptr(b), _ptr(cc),
                                   _ptr(xx), float(alpha), float(beta),
                                   float(x_factor), int(bool(relu)), _ptr(D),
                                   _ptr(Y), _ptr(S),
                                   nthreads or host_threads())
    if rc:
        raise ValueError("orc_gemm_epi_full failed (%d)" % rc)
    return D, Y, S


def _gemm_epi_points(lib, M, N, K, L, A, B, C=None, X=None, *, points, ab="f16", b=None,
                    c=None, x=None, a_major="K", b_major="K", cd_major="N",
                    alpha=1.0, beta=0.0, x_factor=0.0, relu=False, nthreads=None):
    """Oracle at listed (l, m, n) points: returns (D_ref, Y_ref, S) per point."""
    d = _desc(M, N, K, L, a_major, b_major, cd_major, ab, c, x, b)
    a, b = _bits(A, ab), _bits(B, b or ab)
    cc = _bits(C, c) if c else None
    xx = _bits(X, x) if x else None
    _check_sizes(M, N, K, L, a, b, cc, xx)
    pts = np.ascontiguousarray(np.asarray(points, dtype=np.int64).reshape(-1, 3))
    n = pts.shape[0]
    D = np.empty(n, np.float64)
    Y = np.empty(n, np.float64)
    S = np.empty(n, np.float64)
    rc = lib.orc_gemm_epi_points(ctypes.byref(d), _ptr(a), _ptr(b),
                                     _ptr(cc), _ptr(xx), float(alpha),
                                     float(beta), float(x_factor),
                                     int(bool(relu)), n, _ptr(pts),
                                     _ptr(D), _ptr(Y), _ptr(S),
                                     nthreads or host_threads())
    if rc:
        raise ValueError("orc_gemm_epi_points failed (%d)" % rc)
    return D, Y, S


def _check_sizes(M, N, K, L, a, b, c, x):
    if a.size < M * K * L or b.size < N * K * L:
        raise ValueError("A/B smaller than M*K*L / N*K*L")
    for t in (c, x):
        if t is not None and t.size < M * N * L:
            raise ValueError("C/X smaller than M*N*L")


def decode(type_name: str, stored) -> np.ndarray:
    """Exact fp64 value of every stored element."""
    return default().decode(type_name, stored)


def gemm_epi(*a, **kw):
    """Full oracle result: (D_ref, Y_ref, S) as flat float64 arrays laid out
    like C/D (packed batches, L outermost, ``cd_major`` contiguous)."""
    return default().gemm_epi(*a, **kw)


def gemm_epi_points(*a, **kw):
    """Oracle at listed (l, m, n) points: (D_ref, Y_ref, S) per point."""
    return default().gemm_epi_points(*a, **kw)

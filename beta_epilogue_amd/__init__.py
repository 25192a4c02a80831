"""Thin Python binding of libgemm_epi.so, the MI355X fused-epilogue GEMM.

Argument marshalling only: every step of the computation runs in the HIP
kernels of the shared library.  The C entry points keep their names
(``gemm_epi_create``, ``gemm_epi_run``, ...); ``FusedGemm`` adds the
torch-tensor convenience layer (pointers and the current HIP stream).

The library must have been built (``python -m beta_epilogue_amd.build`` or
``__graft_entry__.build()``); importing the binding without it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemm_epi.so")

# Public header constants (include/gemm_epi.h)
GEMM_EPI_OK = 0
GEMM_EPI_ERR_INVALID_ARG = 1
GEMM_EPI_ERR_UNSUPPORTED = 2
GEMM_EPI_ERR_ALIGNMENT = 3
GEMM_EPI_ERR_DEVICE = 4
GEMM_EPI_ERR_LAUNCH = 5
GEMM_EPI_ERR_HOST_ALLOC = 6
GEMM_EPI_STATIC_SCRATCH_BYTES = 64 << 20  # include/gemm_epi.h

DTYPES = {None: 0, "none": 0, "f16": 1, "bf16": 2, "e4m3": 3, "i8": 4,
          "f32": 5, "i32": 6, "e5m2": 7, "u8": 8}
MAJOR = {"K": 0, "M": 1, "N": 2}


class gemm_epi_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("L", ctypes.c_int64),
                ("a_major", ctypes.c_int32), ("b_major", ctypes.c_int32),
                ("cd_major", ctypes.c_int32), ("ab_dtype", ctypes.c_int32),
                ("c_dtype", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("d_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32),
                ("epilogue", ctypes.c_int32), ("b_dtype", ctypes.c_int32),
                ("splits", ctypes.c_int32)]


class gemm_epi_plan(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("lds_bytes", ctypes.c_int32),
                ("cus", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64), ("split_tiles", ctypes.c_int64),
                ("name", ctypes.c_char * 64)]


class GemmEpiError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        self.code = code
        super().__init__("%s: %s (%d): %s" % (where, status_string(code), code,
                                              detail))


_lib = None


def lib():
    """The loaded shared library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgemm_epi.so is not built (%s); run "
                               "`python -m beta_epilogue_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        L.gemm_epi_create.argtypes = [ctypes.POINTER(gemm_epi_desc), ctypes.POINTER(P)]
        L.gemm_epi_create.restype = ctypes.c_int
        L.gemm_epi_create_variant.argtypes = [ctypes.POINTER(gemm_epi_desc), ctypes.c_int,
                                              ctypes.POINTER(P)]
        L.gemm_epi_create_variant.restype = ctypes.c_int
        L.gemm_epi_run.argtypes = [P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                   ctypes.c_float, P]
        L.gemm_epi_run.restype = ctypes.c_int
        L.gemm_epi_run_static.argtypes = L.gemm_epi_run.argtypes
        L.gemm_epi_run_static.restype = ctypes.c_int
        L.gemm_epi_destroy.argtypes = [P]
        L.gemm_epi_destroy.restype = ctypes.c_int
        L.gemm_epi_get_plan.argtypes = [P, ctypes.POINTER(gemm_epi_plan)]
        L.gemm_epi_get_plan.restype = ctypes.c_int
        L.gemm_epi_variant_count.argtypes = []
        L.gemm_epi_variant_count.restype = ctypes.c_int
        L.gemm_epi_variant_name.argtypes = [ctypes.c_int]
        L.gemm_epi_variant_name.restype = ctypes.c_char_p
        L.gemm_epi_status_string.argtypes = [ctypes.c_int]
        L.gemm_epi_status_string.restype = ctypes.c_char_p
        L.gemm_epi_last_error.argtypes = []
        L.gemm_epi_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().gemm_epi_status_string(code).decode()


def last_error() -> str:
    return lib().gemm_epi_last_error().decode()


def _check(code: int, where: str):
    if code != GEMM_EPI_OK:
        raise GemmEpiError(code, where, last_error())


EPILOGUES = {"linear": 0, "relu": 1}


def make_desc(M, N, K, L=1, *, ab="f16", a_major="K", b_major="K",
              cd_major="N", c=None, x=None, d="f32", y=None,
              epilogue="linear", b=None, splits=0) -> gemm_epi_desc:
    """b: B's own type when it differs from A's (the fp8 pairs); splits: 0
    (the library's choice), 1 (no split-K) or the number of K slices."""
    return gemm_epi_desc(M, N, K, L, MAJOR[a_major], MAJOR[b_major],
                         MAJOR[cd_major], DTYPES[ab], DTYPES[c], DTYPES[x],
                         DTYPES[d], DTYPES[y], EPILOGUES[epilogue],
                         DTYPES[b] if b and b != ab else 0, splits)


def gemm_epi_create(desc: gemm_epi_desc) -> int:
    h = ctypes.c_void_p()
    _check(lib().gemm_epi_create(ctypes.byref(desc), ctypes.byref(h)),
           "gemm_epi_create")
    return h.value


def gemm_epi_create_variant(desc: gemm_epi_desc, variant: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().gemm_epi_create_variant(ctypes.byref(desc), variant,
                                         ctypes.byref(h)),
           "gemm_epi_create_variant")
    return h.value


def gemm_epi_run(h: int, A: int, B: int, C: Optional[int], X: Optional[int],
                 D: int, Y: Optional[int], alpha: float, beta: float,
                 x_factor: float, stream: Optional[int]) -> None:
    _check(lib().gemm_epi_run(h, A, B, C, X, D, Y, alpha, beta, x_factor,
                              stream), "gemm_epi_run")


def gemm_epi_run_static(h: int, A: int, B: int, C: Optional[int], X: Optional[int],
                        D: int, Y: Optional[int], alpha: float, beta: float,
                        x_factor: float, stream: Optional[int]) -> None:
    _check(lib().gemm_epi_run_static(h, A, B, C, X, D, Y, alpha, beta, x_factor,
                                     stream), "gemm_epi_run_static")


def gemm_epi_destroy(h: Optional[int]) -> None:
    _check(lib().gemm_epi_destroy(h), "gemm_epi_destroy")


def gemm_epi_get_plan(h: int) -> dict:
    p = gemm_epi_plan()
    _check(lib().gemm_epi_get_plan(h, ctypes.byref(p)), "gemm_epi_get_plan")
    return {"variant": p.variant, "tile_m": p.tile_m, "tile_n": p.tile_n,
            "tile_k": p.tile_k, "threads": p.threads, "grid": p.grid,
            "tiles": p.tiles, "lds_bytes": p.lds_bytes, "cus": p.cus,
            "splits": p.splits, "workspace_bytes": p.workspace_bytes, "split_tiles": p.split_tiles,
            "name": p.name.decode()}


def gemm_epi_variant_count() -> int:
    return lib().gemm_epi_variant_count()


def gemm_epi_variant_name(i: int) -> Optional[str]:
    r = lib().gemm_epi_variant_name(i)
    return None if r is None else r.decode()


class FusedGemm:
    """One problem shape: a handle plus torch-tensor marshalling.

    Tensors are device tensors in the packed layouts of the C header; their
    data pointers and ``torch.cuda.current_stream()`` go straight to
    ``gemm_epi_run``.  No computation happens in Python.
    """

    def __init__(self, M, N, K, L=1, *, ab="f16", a_major="K", b_major="K",
                 cd_major="N", c=None, x=None, d="f32", y=None, variant=-1,
                 epilogue="linear", b=None, splits=0):
        self.desc = make_desc(M, N, K, L, ab=ab, a_major=a_major,
                              b_major=b_major, cd_major=cd_major, c=c, x=x,
                              d=d, y=y, epilogue=epilogue, b=b, splits=splits)
        self.shape = (M, N, K, L)
        self.handle = (gemm_epi_create(self.desc) if variant == -1
                       else gemm_epi_create_variant(self.desc, variant))

    @property
    def plan(self) -> dict:
        return gemm_epi_get_plan(self.handle)

    @staticmethod
    def _ptr(t):
        if t is None:
            return None
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be packed (contiguous)")
        return t.data_ptr()

    def __call__(self, A, B, C=None, X=None, *, D, Y=None, alpha=1.0,
                 beta=0.0, x_factor=0.0, stream=None, static_scratch=False):
        """static_scratch: run through gemm_epi_run_static (no allocation)."""
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        run = gemm_epi_run_static if static_scratch else gemm_epi_run
        run(self.handle, self._ptr(A), self._ptr(B), self._ptr(C),
            self._ptr(X), self._ptr(D), self._ptr(Y), float(alpha),
            float(beta), float(x_factor), sptr)
        return D

    def close(self):
        if self.handle:
            gemm_epi_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

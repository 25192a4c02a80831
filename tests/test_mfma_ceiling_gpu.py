"""The MFMA-ceiling measurement tool (libmfma_ceiling.so, bench.py
--mfma-ceiling) runs every operand type and block shape and reports rates
within the datasheet peaks and clocks within the part's range."""
import ctypes
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# operand type code (gemm_epi.h) -> dense peak of the part, 10^12 per second
PEAKS = {1: 2500.0, 2: 2500.0, 3: 5000.0, 4: 5000.0}


@pytest.mark.gpu
@pytest.mark.parametrize("type_code", sorted(PEAKS))
@pytest.mark.parametrize("block", [32, 16])
def test_ceiling_stream_runs(type_code, block):
    import torch
    torch.cuda.init()
    lib = ctypes.CDLL(os.path.join(ROOT, "beta_epilogue_amd", "libmfma_ceiling.so"))
    fn = lib.mfma_ceiling_run_type
    fn.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double)]
    fn.restype = ctypes.c_int
    for rnd in (0, 1):
        ms, ghz, tf = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
        print("ceiling type %d block %d random %d" % (type_code, block, rnd), flush=True)
        assert fn(type_code, block, rnd, 4000, 1, ctypes.byref(ms), ctypes.byref(ghz), ctypes.byref(tf)) == 0
        assert ms.value > 0.0
        assert 0.5 < ghz.value < 3.0
        assert 0.05 * PEAKS[type_code] < tf.value < 1.05 * PEAKS[type_code]


def test_ceiling_rejects_unknown_type_and_block():
    """Argument checks happen before any HIP call, so they run without a GPU."""
    lib = ctypes.CDLL(os.path.join(ROOT, "beta_epilogue_amd", "libmfma_ceiling.so"))
    fn = lib.mfma_ceiling_run_type
    fn.restype = ctypes.c_int
    ms, ghz, tf = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
    for t, b in ((0, 32), (5, 32), (1, 8), (4, 64)):
        assert fn(t, b, 0, 8, 1, ctypes.byref(ms), ctypes.byref(ghz), ctypes.byref(tf)) != 0

"""gemm_epi_run_static: the allocation-free run (the workspace -- split-K
partial sums, uint8 sums and copies, fp16 copies of widened fp8 -- in the
library's static device array) against gemm_epi_run (the handle's own
workspace), bit for bit, on calls in a row, each smaller than the one
before."""
import sys

import numpy as np
import pytest
import torch

import synth
from parity import parity_full, run_gpu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    (synth.CONFIGS[2].replace(name="static_f16_cxdy", M=512, N=520, K=4096, L=2, seed=7400), 8),
    (synth.CONFIGS[3].replace(name="static_i8_small", M=256, N=272, K=1024, L=1, seed=7410), 3),
    # uint8: the row and column sums in the static array (no split)
    (synth.CONFIGS[3].replace(name="static_u8_smaller", M=128, N=144, K=512, L=1, ab="u8",
                              dist_ab="u8full", seed=7420), 0),
    # fp8 with fp32 outputs: split-K partial sums, then the fp16 copies of A and B
    (synth.CONFIGS[4].replace(name="static_e4m3_f32_widened", M=96, N=128, K=512, L=1, c="f32",
                              d="f32", seed=7430), 2),
]


def test_run_static_matches_run_twice_second_smaller():
    import beta_epilogue_amd as ge
    for p, splits in CASES:
        _say("case", p.name, p.M, p.N, p.K, p.L, "splits", splits)
        ins = synth.make_inputs(p)
        D1, Y1, plan = run_gpu(p, ins, splits=splits)
        D2, Y2, plan2 = run_gpu(p, ins, splits=splits, static_scratch=True)
        assert plan["splits"] == max(splits, 1) and plan2["splits"] == max(splits, 1)
        assert plan["workspace_bytes"] <= ge.GEMM_EPI_STATIC_SCRATCH_BYTES
        assert torch.equal(D1.view(torch.uint8), D2.view(torch.uint8)), "static run differs"
        if Y1 is not None:
            assert torch.equal(Y1.view(torch.uint8), Y2.view(torch.uint8))
        (ed, ey), _ = parity_full(p, ins=ins, exact=p.ab == "i8", splits=splits)
        _say("  err D %.3g Y %.3g" % (ed, ey))


def test_run_static_refuses_a_workspace_beyond_its_array():
    import beta_epilogue_amd as ge
    # 16 slices of 1024 x 1024 fp32 partial sums: exactly 64 MiB fits; 2048 x 1024 does not
    g = ge.FusedGemm(2048, 1024, 16384, ab="f16", d="f32", splits=16)
    assert g.plan["workspace_bytes"] > ge.GEMM_EPI_STATIC_SCRATCH_BYTES
    a = torch.zeros(2048 * 16384, dtype=torch.float16, device="cuda")
    b = torch.zeros(1024 * 16384, dtype=torch.float16, device="cuda")
    d = torch.zeros(2048 * 1024, dtype=torch.float32, device="cuda")
    with pytest.raises(ge.GemmEpiError) as e:
        g(a, b, D=d, static_scratch=True)
    assert e.value.code == ge.GEMM_EPI_ERR_UNSUPPORTED
    g.close()

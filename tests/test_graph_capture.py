"""gemm_epi_run_static under HIP graph capture (torch.cuda.graph): the
allocation-free run recorded once and replayed several times, with eager
runs sharing the static workspace between the replays; every replay must
equal the eager result bit for bit."""
import sys

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # no workspace
    (synth.CONFIGS[2].replace(name="graph_f16_cxdy", M=520, N=264, K=392, L=2, seed=7600), 0),
    # split-K partial sums in the static array, then the reduction kernel
    (synth.CONFIGS[2].replace(name="graph_f16_splitk", M=256, N=264, K=4096, L=1, seed=7610), 4),
    # uint8 with an M-major A: the zeroing kernel, both preparation passes
    (synth.CONFIGS[3].replace(name="graph_u8_mmajor", M=272, N=256, K=640, L=2, ab="u8",
                              dist_ab="u8full", seed=7620), 0),
    # fp8 with an fp32 output: the widening passes, then the fp16 kernel
    (synth.CONFIGS[4].replace(name="graph_e4m3_f32", M=264, N=256, K=512, L=1, c="f32", d="f32",
                              seed=7630), 0),
    # whole-K rounds, then the last round's tiles in K slices (289 tiles on 256 CUs)
    (synth.CONFIGS[2].replace(name="graph_f16_split_last_round", M=4352, N=4352, K=4096, L=1,
                              seed=7640), 0),
    # a small problem on 128x128 tiles whose K is split (workspace slots of the smaller tile)
    (synth.CONFIGS[2].replace(name="graph_f16_small_tiles_split", M=1024, N=1024, K=8192, L=1,
                              seed=7650), 0),
]


@pytest.mark.parametrize("p,splits", CASES, ids=[c[0].name for c in CASES])
def test_run_static_replays_match_eager(p, splits):
    import beta_epilogue_amd as ge
    _say("case", p.name, p.M, p.N, p.K, p.L, "splits", splits)
    ins = synth.make_inputs(p)
    dev = {k: (v.cuda() if v is not None else None) for k, v in ins.items()}
    g = ge.FusedGemm(p.M, p.N, p.K, p.L, ab=p.ab, a_major=p.a_major, b_major=p.b_major,
                     cd_major=p.cd_major, c=p.c, x=p.x, d=p.d, y=p.y, splits=splits)
    assert g.plan["workspace_bytes"] <= ge.GEMM_EPI_STATIC_SCRATCH_BYTES
    if p.name.endswith("split_last_round"):
        assert 0 < g.plan["split_tiles"] < g.plan["tiles"] and g.plan["splits"] > 1, g.plan
    if p.name.endswith("small_tiles_split"):
        assert "128x128" in g.plan["name"] and g.plan["splits"] > 1 and g.plan["workspace_bytes"] > 0, g.plan
    shape = p.storage_shape("D")

    def outputs():
        D = torch.empty(shape, dtype=synth.TORCH_DTYPE[p.d], device="cuda")
        Y = torch.empty(shape, dtype=synth.TORCH_DTYPE[p.y], device="cuda") if p.y else None
        return D, Y

    def run(D, Y):
        g(dev["A"], dev["B"], dev["C"], dev["X"], D=D, Y=Y, alpha=p.alpha, beta=p.beta,
          x_factor=p.x_factor, static_scratch=True)

    De, Ye = outputs()
    run(De, Ye)  # eager reference (also the warm-up before capture)
    torch.cuda.synchronize()

    Dg, Yg = outputs()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(Dg, Yg)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(Dg, Yg)
    torch.cuda.synchronize()

    Dt, Yt = outputs()
    for rep in range(3):
        Dg.zero_()
        if Yg is not None:
            Yg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Dg.view(torch.uint8), De.view(torch.uint8)), "replay %d: D differs" % rep
        if Ye is not None:
            assert torch.equal(Yg.view(torch.uint8), Ye.view(torch.uint8)), "replay %d: Y differs" % rep
        run(Dt, Yt)  # eager work on the same static workspace between replays
        torch.cuda.synchronize()
        assert torch.equal(Dt.view(torch.uint8), De.view(torch.uint8))
    _say("  plan", g.plan["name"], "splits", g.plan["splits"], "workspace", g.plan["workspace_bytes"])
    del graph
    g.close()

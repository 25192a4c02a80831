"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Every test here needs an MI355X and the built library.  Inputs come from the
seeded generators in ``synth``; expected values only ever come from the
oracle.  Each case prints its name and shape before touching the GPU.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from parity import parity_full, parity_sampled, run_gpu, to_f64

pytestmark = pytest.mark.gpu

CFG = synth.CONFIGS


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def small(p, M, N, K, L=None):
    return p.replace(name=p.name + "_small", M=M, N=N, K=K, L=L or p.L)


# Scaled-down versions of the five workloads: same types, layouts, scalars and
# value distributions; several 256x256 tiles with ragged M, N and K tails.
SMALL_CASES = [
    (CFG[0], True),                                  # 128^3, exact by construction
    (small(CFG[1], 592, 528, 392), False),           # bf16 -> f32
    (small(CFG[2], 600, 520, 392), False),           # f16, C X D Y
    (small(CFG[3], 592, 528, 400, L=2), False),      # int8, A M-major, batched
    (small(CFG[4], 600, 528, 400), False),           # e4m3 -> f16
]


@pytest.mark.parametrize("p,exact", SMALL_CASES, ids=[c[0].name for c in SMALL_CASES])
def test_parity_small_full_oracle(p, exact):
    _say("case", p.name, p.M, p.N, p.K, p.L)
    (ed, ey), plan = parity_full(p, exact=exact)
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5], ids=[c.name for c in CFG[1:6]])
def test_parity_full_size_sampled(i):
    """The benchmark shapes, in the launch configuration the bench times."""
    p = CFG[i]
    _say("case", p.name, p.M, p.N, p.K, p.L)
    (ed, ey), plan, npts = parity_sampled(p)
    _say("  plan", plan["name"], "grid", plan["grid"], "points", npts,
         "err D %.3g Y %.3g" % (ed, ey))


def test_config0_bit_exact():
    p = CFG[0]
    _say("case", p.name)
    (ed, ey), plan = parity_full(p, exact=True)
    assert ed == 0.0


EDGE = [
    # 4-byte C/D without X and Y, lines 4 mod 8 elements long (each line
    # ends half-way through a 32-byte group)
    CFG[3].replace(name="i32_no_xy_n_4mod8", M=136, N=260, K=128, L=2, a_major="K", seed=6050),
    CFG[3].replace(name="i32_no_xy_cdm_m_4mod8", M=260, N=136, K=128, L=1, a_major="K", cd_major="M",
                   beta=-2.0, seed=6060),
    CFG[1].replace(name="f32_no_xy_n_4mod8_relu", M=200, N=268, K=136, epilogue="relu", beta=-1.0, seed=6070),
    CFG[1].replace(name="f32_no_xy_cdm_m_4mod8", M=268, N=200, K=136, cd_major="M", seed=6080),
    CFG[2].replace(name="one_row", M=1, N=8, K=8, L=1),
    CFG[2].replace(name="tiny_batched", M=3, N=16, K=24, L=3),
    CFG[2].replace(name="k_tail_only", M=256, N=256, K=72, L=1),
    CFG[2].replace(name="cd_mmajor_f16", M=264, N=136, K=136, L=2, cd_major="M"),
    CFG[1].replace(name="cd_mmajor_f32", M=520, N=260, K=200, cd_major="M", seed=6100),
    CFG[1].replace(name="bf16_out", M=300, N=264, K=128, d="bf16", c="bf16", seed=6200),
    CFG[1].replace(name="y_only_f32", M=130, N=260, K=64, y="f32", beta=0.0, c=None,
                   seed=6300),
    CFG[4].replace(name="e4m3_mmajor_cd", M=264, N=296, K=160, cd_major="M", seed=6400),
    CFG[4].replace(name="e4m3_xy", M=260, N=264, K=256, x="bf16", y="f32", x_factor=-1.5,
                   seed=6500),
    CFG[3].replace(name="i8_kmajor_xy", M=260, N=264, K=160, L=1, a_major="K", x="i32",
                   y="i32", alpha=-3.0, beta=2.0, x_factor=5.0, dist_x="i1000", seed=6600),
    CFG[3].replace(name="i8_mmajor_cdm", M=272, N=260, K=176, L=2, cd_major="M", seed=6700),
    CFG[3].replace(name="i8_mmajor_ktail", M=48, N=40, K=48, L=1, seed=6800),
    CFG[2].replace(name="f16_large_k", M=256, N=512, K=4104, seed=6900),
    # N-major f16 C/X/D/Y with both tile extents cut: 8-element lane groups
    # past N and rows past M
    CFG[2].replace(name="f16_ragged_mn", M=300, N=392, K=96, seed=7000),
    # mixed C/X/D/Y types (general epilogue), ragged N
    CFG[1].replace(name="mixed_types_ragged", M=300, N=264, K=128, c="f32", x="bf16",
                   y="bf16", x_factor=0.5, seed=7060),
    # M-major A and N-major B (transposing LDS reads): ragged M, N and K tails,
    # K shorter than one K tile, tiny extents, every type
    CFG[2].replace(name="mn_f16_ktail", M=264, N=136, K=72, a_major="M", b_major="N", seed=7100),
    CFG[2].replace(name="mn_f16_tiny", M=8, N=16, K=8, L=3, a_major="M", b_major="N", seed=7110),
    CFG[1].replace(name="kn_bf16_cdm", M=300, N=264, K=200, b_major="N", cd_major="M", seed=7120),
    CFG[1].replace(name="mk_bf16_ragged", M=200, N=300, K=264, a_major="M", seed=7125),
    CFG[4].replace(name="mk_e4m3", M=272, N=296, K=176, a_major="M", seed=7130),
    CFG[4].replace(name="kn_e4m3_cdm", M=296, N=272, K=144, b_major="N", cd_major="M", seed=7135),
    CFG[4].replace(name="mn_e4e5_pair_widened", M=272, N=288, K=160, a_major="M", b_major="N",
                   b_ab="e5m2", dist_b="e5m2tab", seed=7140),
    CFG[3].replace(name="mn_i8_short_k", M=272, N=272, K=48, L=2, b_major="N", seed=7150),
    CFG[3].replace(name="kn_i8_xy", M=260, N=272, K=272, L=1, a_major="K", b_major="N",
                   x="i32", y="i32", alpha=-3.0, beta=2.0, x_factor=5.0, dist_x="i1000",
                   seed=7160),
    # int32 outputs with unit scalars take the adds-only epilogue: C skipped
    # (beta 0) with X added, and both added; a scalar of 2 takes the
    # multiplying one
    CFG[3].replace(name="kk_i8_unit_x_no_c", M=264, N=272, K=208, L=2, a_major="K",
                   x="i32", y="i32", alpha=1.0, beta=0.0, x_factor=1.0, dist_x="i1000",
                   seed=7170),
    CFG[3].replace(name="mk_i8_unit_c_x_cdm", M=272, N=264, K=144, L=1, cd_major="M",
                   x="i32", alpha=1.0, beta=1.0, x_factor=1.0, dist_x="i1000", seed=7180),
    CFG[3].replace(name="mk_i8_x2_not_unit", M=272, N=264, K=144, L=1,
                   x="i32", alpha=1.0, beta=1.0, x_factor=2.0, dist_x="i1000", seed=7190),
]


def test_general_epilogue_both_block_shapes_ragged_n():
    """Mixed C/X/D/Y types run the mixed-type epilogue on the 16x16-block
    kernels (256x256 and the 128x128 tiles the plan takes for this small
    problem) and on a 32x32-block variant alike (N-major: 16x16; M-major
    C/D: 32x32; forced 32x32 for f16 N-major): linear and ReLU forms, a
    ragged N tile, with and without Y, batched.  (M = 191, N = 344 with f32
    C and bf16 D/Y once gave wrong values with 16x16 blocks.)"""
    import beta_epilogue_amd as ge
    names = [ge.gemm_epi_variant_name(i) for i in range(ge.gemm_epi_variant_count())]
    for cd, v in (("N", "bf16_kk_n_256x256_r128_w4_s2_b16"), ("N", "bf16_kk_n_128x128_r128_w4_s2_b16"),
                  ("M", "bf16_kk_m_256x256_r128_w4_s2_q2")):
        for epi in ("linear", "relu"):
            for y in (None, "bf16"):
                p = CFG[1].replace(name="general_%s_%s_%s" % (v, epi, y), M=192 if cd == "M" else 191,
                                   N=344, K=200, L=2, c="f32", x="bf16", y=y,
                                   d="bf16" if y else "f32", x_factor=0.5, cd_major=cd,
                                   beta=-1.0 if epi == "relu" else 1.0, epilogue=epi, seed=7070)
                _say("case", p.name)
                _, plan = parity_full(p, variant=names.index(v))
                assert plan["name"] == v, plan["name"]
    # the plan's own choice for this size: the 128x128 tiles (N-major), the
    # 256x256 default (M-major C/D, no 128x128 kernel)
    for cd, v in (("N", "bf16_kk_n_128x128_r128_w4_s2_b16"), ("M", "bf16_kk_m_256x256_r128_w4_s2_q2")):
        p = CFG[1].replace(name="general_auto_" + cd, M=192, N=344, K=200, L=2, c="f32", x="bf16", y="bf16",
                           d="bf16", x_factor=0.5, cd_major=cd, seed=7072)
        _, plan = parity_full(p)
        assert plan["name"] == v, plan["name"]
    v = "f16_kk_n_256x256_r128_w4_s2_q2"
    p = CFG[2].replace(name="general_" + v, M=191, N=344, K=200, L=2, c="f32", x="bf16",
                       y="f16", d="bf16", x_factor=0.5, seed=7071)
    _, plan = parity_full(p, variant=names.index(v))
    assert plan["name"] == v


@pytest.mark.parametrize("p", EDGE, ids=[e.name for e in EDGE])
def test_parity_edge_cases(p):
    _say("case", p.name, p.M, p.N, p.K, p.L, p.cd_major)
    (ed, ey), plan = parity_full(p)
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


# The ReLU form D = max(0, alpha*A.B^T + beta*C) + x_factor*X: mixed-sign
# sums so both sides of the clamp occur; typed epilogues (f16, f32, int32)
# and the mixed-type one, both majornesses.
RELU = [
    small(CFG[2], 600, 520, 392).replace(name="relu_f16_cxdy", epilogue="relu", seed=7200),
    small(CFG[2], 264, 392, 136).replace(name="relu_f16_mmajor", cd_major="M",
                                         epilogue="relu", seed=7300),
    small(CFG[1], 592, 528, 392).replace(name="relu_bf16_f32", alpha=1.0, beta=-1.0,
                                         epilogue="relu", seed=7400),
    small(CFG[3], 592, 528, 400, L=2).replace(name="relu_i8_mmajorA", beta=-1.0,
                                              epilogue="relu", seed=7500),
    CFG[3].replace(name="relu_i8_kmajor_xy", M=260, N=264, K=160, L=1, a_major="K",
                   x="i32", y="i32", alpha=-3.0, beta=2.0, x_factor=5.0, dist_x="i1000",
                   epilogue="relu", seed=7600),
    CFG[4].replace(name="relu_e4m3_mixed", M=260, N=264, K=256, x="bf16", y="f32",
                   x_factor=-1.5, beta=-1.0, epilogue="relu", seed=7700),
]


@pytest.mark.parametrize("p", RELU, ids=[e.name for e in RELU])
def test_parity_relu(p):
    _say("case", p.name, p.M, p.N, p.K, p.L, p.cd_major)
    (ed, ey), plan = parity_full(p)
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


def test_parity_relu_full_size_sampled():
    """The 8192^3 fp16 workload in the ReLU form, at the bench's launch."""
    p = CFG[2].replace(name="f16_8192_fused_cxdy_relu", epilogue="relu")
    _say("case", p.name)
    (ed, ey), plan, npts = parity_sampled(p)
    _say("  plan", plan["name"], "points", npts, "err D %.3g Y %.3g" % (ed, ey))


# D == C in place: bit-identical to the out-of-place run, and within the bar
# of the oracle, for typed (f16, int32) and mixed-type epilogues.  Every C
# element is loaded by the lane that later stores its D (the example's
# epilogue: all loads before any store).
INPLACE = [
    small(CFG[2], 600, 520, 392).replace(name="inplace_f16", seed=7800),
    small(CFG[2], 264, 392, 136).replace(name="inplace_f16_relu_mmajor", cd_major="M",
                                         epilogue="relu", seed=7850),
    small(CFG[3], 592, 528, 400, L=2).replace(name="inplace_i32", seed=7900),
    CFG[1].replace(name="inplace_mixed", M=300, N=264, K=128, d="f32", c="f32", x="bf16",
                   x_factor=0.5, seed=7950),
]


@pytest.mark.parametrize("p", INPLACE, ids=[e.name for e in INPLACE])
def test_inplace_d_is_c(p):
    import beta_epilogue_amd as ge
    _say("case", p.name, p.M, p.N, p.K, p.L, p.cd_major)
    ins = synth.make_inputs(p)
    D_out, Y_out, _ = run_gpu(p, ins)
    dev = {k: (v.cuda() if v is not None else None) for k, v in ins.items()}
    g = ge.FusedGemm(p.M, p.N, p.K, p.L, ab=p.ab, a_major=p.a_major, b_major=p.b_major,
                     cd_major=p.cd_major, c=p.c, x=p.x, d=p.d, y=p.y, epilogue=p.epilogue)
    CD = dev["C"].clone()
    Y = torch.empty_like(Y_out, device="cuda") if p.y else None
    g(dev["A"], dev["B"], CD, dev["X"], D=CD, Y=Y, alpha=p.alpha, beta=p.beta,
      x_factor=p.x_factor)
    torch.cuda.synchronize()
    g.close()
    assert torch.equal(CD.cpu().view(torch.uint8), D_out.view(torch.uint8)), "in place != out of place"
    if p.y:
        assert torch.equal(Y.cpu().view(torch.uint8), Y_out.view(torch.uint8))
    (ed, ey), _ = parity_full(p, ins=ins)
    _say("  err D %.3g Y %.3g" % (ed, ey))


def test_aliasing_rules():
    """Every overlap other than D == C (with C read, same type) is refused
    before launch: D or Y on X, Y on C, Y on D, D on an unread C."""
    import beta_epilogue_amd as ge
    p = small(CFG[2], 256, 256, 64)
    ins = synth.make_inputs(p)
    dev = {k: (v.cuda() if v is not None else None) for k, v in ins.items()}
    g = ge.FusedGemm(p.M, p.N, p.K, p.L, ab=p.ab, c=p.c, x=p.x, d=p.d, y=p.y)
    D = torch.empty_like(dev["C"])
    for kw in (dict(D=dev["X"], Y=D), dict(D=D, Y=dev["X"]), dict(D=D, Y=dev["C"]),
               dict(D=D, Y=D)):
        with pytest.raises(ge.GemmEpiError) as e:
            g(dev["A"], dev["B"], dev["C"], dev["X"], alpha=p.alpha, beta=p.beta,
              x_factor=p.x_factor, **kw)
        assert e.value.code == ge.GEMM_EPI_ERR_INVALID_ARG
    # D == C with beta == 0 (C not read) is not an in-place update
    with pytest.raises(ge.GemmEpiError) as e:
        g(dev["A"], dev["B"], dev["C"], dev["X"], D=dev["C"], Y=D, alpha=1.0, beta=0.0,
          x_factor=p.x_factor)
    assert e.value.code == ge.GEMM_EPI_ERR_INVALID_ARG
    g.close()
    # D == C with a C of another element type is refused too
    g = ge.FusedGemm(256, 256, 64, ab="f16", c="f32", d="f16")
    c32 = torch.zeros(256 * 256 * 2, dtype=torch.float16, device="cuda")
    with pytest.raises(ge.GemmEpiError) as e:
        g(dev["A"], dev["B"], c32, D=c32, alpha=1.0, beta=1.0)
    assert e.value.code == ge.GEMM_EPI_ERR_INVALID_ARG
    g.close()


# fp8 e5m2 A/B (format selectors 1/1 of the f8f6f4 MFMA): the e4m3 workload's
# shapes and outputs with e5m2 values of |v| <= 4; the f32-output case runs
# widened (fp16 copies, fp16 kernel).
E5M2 = [
    small(CFG[4], 600, 528, 400).replace(name="e5m2_f16out", ab="e5m2", dist_ab="e5m2tab",
                                         seed=8100),
    CFG[4].replace(name="e5m2_mmajor_cd", M=264, N=296, K=160, cd_major="M", ab="e5m2",
                   dist_ab="e5m2tab", seed=8200),
    CFG[4].replace(name="e5m2_f32_xy", M=260, N=264, K=256, d="f32", c="f32", x="bf16",
                   y="f32", x_factor=-1.5, ab="e5m2", dist_ab="e5m2tab", seed=8300),
    CFG[4].replace(name="e5m2_relu", M=260, N=264, K=256, ab="e5m2", dist_ab="e5m2tab",
                   beta=-1.0, epilogue="relu", seed=8400),
]


@pytest.mark.parametrize("p", E5M2, ids=[e.name for e in E5M2])
def test_parity_e5m2(p):
    _say("case", p.name, p.M, p.N, p.K, p.L, p.cd_major)
    (ed, ey), plan = parity_full(p)
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


# fp8 pairs: A e4m3 with B e5m2 and the reverse (per-operand format
# selectors, or each operand widened by its own format with fp32 outputs).
F8PAIRS = [
    small(CFG[4], 600, 528, 400).replace(name="e4m3_x_e5m2", b_ab="e5m2", dist_b="e5m2tab",
                                         seed=8600),
    small(CFG[4], 600, 528, 400).replace(name="e5m2_x_e4m3", ab="e5m2", dist_ab="e5m2tab",
                                         b_ab="e4m3", dist_b="e4m3tab", seed=8700),
    CFG[4].replace(name="e4m3_x_e5m2_f32_xy", M=260, N=264, K=256, d="f32", c="f32", x="bf16",
                   y="f32", x_factor=-1.5, b_ab="e5m2", dist_b="e5m2tab", seed=8800),
    CFG[4].replace(name="e4m3_x_e5m2_mmajor", M=264, N=296, K=160, cd_major="M", b_ab="e5m2",
                   dist_b="e5m2tab", seed=8900),
    CFG[4].replace(name="e5m2_x_e4m3_mmajor_relu", M=264, N=296, K=160, cd_major="M",
                   ab="e5m2", dist_ab="e5m2tab", b_ab="e4m3", dist_b="e4m3tab", beta=-1.0,
                   epilogue="relu", seed=8950),
]


@pytest.mark.parametrize("p", F8PAIRS, ids=[e.name for e in F8PAIRS])
def test_parity_fp8_pairs(p):
    _say("case", p.name, p.M, p.N, p.K, p.L, p.ab, p.b_ab)
    (ed, ey), plan = parity_full(p)
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


def test_parity_e5m2_full_size_sampled():
    p = CFG[4].replace(name="e5m2_8192_f16out", ab="e5m2", dist_ab="e5m2tab", seed=8500)
    _say("case", p.name)
    (ed, ey), plan, npts = parity_sampled(p)
    _say("  plan", plan["name"], "points", npts, "err D %.3g Y %.3g" % (ed, ey))


# fp8 inputs with fp32 outputs run widened: fp16 copies of A and B (exact)
# and an fp16 kernel; held to the fp32 bar, 1e-5, like every fp32 output.
FP8_F32 = [
    CFG[4].replace(name="e4m3_f32_out", M=600, N=528, K=400, d="f32", c="f32", seed=8910),
    CFG[4].replace(name="e4m3_f32_y_only", M=264, N=296, K=1024, d="f16", y="f32", seed=8920),
    CFG[4].replace(name="e4m3_f32_mmajor", M=264, N=296, K=160, cd_major="M", d="f32",
                   c="f32", x="f32", x_factor=0.75, y="f32", seed=8930),
    CFG[4].replace(name="e5m2_f32_out_k_tail", M=300, N=264, K=144, ab="e5m2",
                   dist_ab="e5m2tab", d="f32", c="f16", seed=8940),
]


@pytest.mark.parametrize("p", FP8_F32, ids=[e.name for e in FP8_F32])
def test_parity_fp8_fp32_outputs(p):
    _say("case", p.name, p.M, p.N, p.K, p.L, p.ab, p.d, p.y)
    (ed, ey), plan = parity_full(p)
    # the fp16 kernel of the layout, on fp16 copies of A and B in the workspace
    up = lambda x: (x + 255) // 256 * 256
    copies = up(p.L * p.M * p.K * 2) + up(p.L * p.N * p.K * 2)
    assert plan["name"].startswith("f16_") and plan["workspace_bytes"] >= copies, plan
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


def test_parity_more_tiles_than_compute_units():
    """Whole-output parity on a launch with more tiles (320) than workgroups:
    every workgroup walks several tiles of several batches."""
    p = CFG[2].replace(name="f16_2048x5_k64", M=2048, N=2048, K=64, L=5, seed=8990)
    _say("case", p.name)
    (ed, ey), plan = parity_full(p)
    assert plan["tiles"] > plan["grid"], plan
    _say("  plan", plan["name"], "grid", plan["grid"], "tiles", plan["tiles"],
         "err D %.3g Y %.3g" % (ed, ey))


# Split K: the K range in slices whose fp32 (int32) partial sums a second
# kernel adds before the epilogue.  Forced slice counts on small problems
# (every output type path, both C/D majornesses, M/N-major operands, int8
# exact), and the library's own choice on a few-tile, long-K shape.
SPLITK = [
    (CFG[2].replace(name="splitk3_f16_cxdy", M=300, N=264, K=1000, seed=7300), 3),
    (CFG[2].replace(name="splitk2_f16_relu_cdm", M=264, N=392, K=520, cd_major="M",
                    epilogue="relu", seed=7310), 2),
    (CFG[1].replace(name="splitk5_bf16_mixed_l2", M=200, N=264, K=1288, L=2, c="f32", x="bf16",
                    y="bf16", x_factor=0.5, seed=7320), 5),
    (CFG[3].replace(name="splitk4_i8_mmajorA", M=272, N=272, K=2048, L=2, seed=7330), 4),
    (CFG[4].replace(name="splitk3_e4m3_kn", M=272, N=288, K=1152, b_major="N", seed=7340), 3),
    (CFG[4].replace(name="splitk2_f8w_f32", M=272, N=288, K=768, d="f32", c="f32", y="f32",
                    seed=7350), 2),
]


@pytest.mark.parametrize("p,splits", SPLITK, ids=[c[0].name for c in SPLITK])
def test_parity_split_k(p, splits):
    _say("case", p.name, p.M, p.N, p.K, p.L, "splits", splits)
    (ed, ey), plan = parity_full(p, exact=p.ab == "i8", splits=splits)
    assert plan["splits"] == splits and plan["split_tiles"] == plan["tiles"], plan
    # one tile-sized slot of partial sums per slice of every tile, then (fp8
    # with fp32 outputs, widened) the fp16 copies of A and B, each part at a
    # 256-byte boundary
    up = lambda x: (x + 255) // 256 * 256
    ws = splits * plan["tiles"] * plan["tile_m"] * plan["tile_n"] * 4
    if p.ab in ("e4m3", "e5m2") and "f32" in (p.d, p.y):
        ws = up(ws) + up(p.L * p.M * p.K * 2) + up(p.L * p.N * p.K * 2)
    assert plan["workspace_bytes"] == ws
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


def test_split_k_chosen_for_few_long_tiles():
    """512 x 512 x 8192: sixteen 128x128 output tiles (four of 256x256), so
    the library splits K (16 slices of eight K tiles) and fills the GPU;
    whole-output parity."""
    p = CFG[2].replace(name="splitk_auto_512", M=512, N=512, K=8192, seed=7360)
    _say("case", p.name)
    (ed, ey), plan = parity_full(p)
    assert plan["tile_m"] == plan["tile_n"] == 128 and plan["tiles"] == 16, plan
    assert plan["splits"] == 16 and plan["grid"] == 256 and plan["split_tiles"] == 16, plan
    _say("  plan", plan["name"], "splits", plan["splits"], "err D %.3g Y %.3g" % (ed, ey))


# Small problems: when 256x256 tiles would fill at most a quarter of the
# compute units, the plan takes the 128x128-tile kernel of the layout
# (K-major A and B, N-major C/D) where one is built.
SMALL = [
    CFG[2].replace(name="small_f16_cxdy", M=776, N=648, K=520, seed=7700),
    CFG[1].replace(name="small_bf16_f32_l3", M=392, N=264, K=1032, L=3, seed=7710),
    CFG[3].replace(name="small_i8_kk", M=520, N=392, K=1040, L=2, a_major="K", seed=7720),
    CFG[4].replace(name="small_e4m3_f16", M=392, N=520, K=1056, seed=7730),
    CFG[4].replace(name="small_e4m3_f32_widened", M=392, N=264, K=528, c="f32", d="f32", seed=7740),
]


@pytest.mark.parametrize("p", SMALL, ids=[e.name for e in SMALL])
def test_parity_small_problem_tiles(p):
    _say("case", p.name, p.M, p.N, p.K, p.L)
    (ed, ey), plan = parity_full(p, exact=p.ab == "i8")
    assert plan["tile_m"] == plan["tile_n"] == 128 and "_128x128_" in plan["name"], plan
    _say("  plan", plan["name"], "tiles", plan["tiles"], "splits", plan["splits"], "err D %.3g Y %.3g" % (ed, ey))


# A partial last round more than half full (so not split) with 256x256
# tiles: the plan takes 192x256 tiles where they fill the rounds better.
PARTIAL_ROUND = [
    CFG[2].replace(name="round_f16_3000", M=3000, N=3000, K=520, seed=7750),
    CFG[1].replace(name="round_bf16_f32_3000x2960", M=3000, N=2960, K=1032, seed=7760),
]


@pytest.mark.parametrize("p", PARTIAL_ROUND, ids=[e.name for e in PARTIAL_ROUND])
def test_parity_partial_round_tiles(p):
    _say("case", p.name, p.M, p.N, p.K, p.L)
    (ed, ey), plan, npts = parity_sampled(p, sub=32)
    assert plan["tile_m"] == 192 and plan["tile_n"] == 256 and plan["splits"] == 1, plan
    assert plan["tiles"] == -(-p.M // 192) * -(-p.N // 256) * p.L
    _say("  plan", plan["name"], "tiles", plan["tiles"], "points", npts, "err D %.3g Y %.3g" % (ed, ey))


# A partial round that 128x256 tiles fill in one round: fp16 with a ragged K
# tail, int8 with K-major A and ragged M and N, e4m3.
WIDE_TILE = [
    CFG[2].replace(name="wide_f16_2560", M=2560, N=2560, K=1032, seed=7770),
    CFG[3].replace(name="wide_i8_kk_2568x2544", M=2568, N=2544, K=2048, L=1, a_major="K", seed=7780),
    CFG[4].replace(name="wide_e4m3_2552x2560", M=2552, N=2560, K=1024, seed=7790),
]


@pytest.mark.parametrize("p", WIDE_TILE, ids=[e.name for e in WIDE_TILE])
def test_parity_wide_tiles(p):
    _say("case", p.name, p.M, p.N, p.K, p.L)
    (ed, ey), plan, npts = parity_sampled(p, sub=32)
    assert plan["tile_m"] == 128 and plan["tile_n"] == 256, plan
    assert plan["tiles"] == -(-p.M // 128) * -(-p.N // 256) * p.L
    _say("  plan", plan["name"], "tiles", plan["tiles"], "points", npts, "err D %.3g Y %.3g" % (ed, ey))


def test_small_tiles_not_chosen_beyond_a_quarter_of_the_gpu():
    import beta_epilogue_amd as ge
    g = ge.FusedGemm(3072, 3072, 3072, ab="f16", c="f16", x="f16", d="f16", y="f16")
    assert g.plan["tile_m"] == 192, g.plan  # 144 tiles of 256x256: 192 of 192x256
    g.close()
    g = ge.FusedGemm(4096, 4096, 4096, ab="f16", c="f16", x="f16", d="f16", y="f16")
    assert g.plan["tile_m"] == g.plan["tile_n"] == 256, g.plan  # one whole round
    g.close()
    g = ge.FusedGemm(3584, 3584, 3584, ab="f16", c="f16", x="f16", d="f16", y="f16")
    assert g.plan["tile_m"] == g.plan["tile_n"] == 256, g.plan  # 192x256: 266 tiles, a 10-tile round
    g.close()
    g = ge.FusedGemm(2048, 2048, 2048, ab="f16", c="f16", x="f16", d="f16", y="f16")
    assert g.plan["tile_m"] == 128 and g.plan["tiles"] == 256, g.plan  # 64 tiles of 256x256
    g.close()
    g = ge.FusedGemm(512, 512, 512, ab="f16", d="f16", cd_major="M")
    assert g.plan["tile_m"] == 256, g.plan  # no 128x128 kernel for M-major C/D
    g.close()


def test_split_k_not_chosen_when_tiles_fill_the_gpu():
    import beta_epilogue_amd as ge
    g = ge.FusedGemm(8192, 8192, 8192, ab="f16", c="f16", x="f16", d="f16", y="f16")
    assert g.plan["splits"] == 1 and g.plan["workspace_bytes"] == 0 and g.plan["split_tiles"] == 0
    g.close()


# A last round of tiles that would leave most compute units idle: whole-K
# rounds of the other tiles, then the last round's tiles in K slices (the
# library's choice).  Ragged edges, both C/D majornesses, int8 exact, a
# batched bf16 -> fp32 case.  Sampled parity with a point in every 32 x 32
# block of every output tile (a slot added to the wrong tile or at a wrong
# pitch fails), whole edge rows and columns, and random points.
SPLIT_TAIL = [
    CFG[2].replace(name="tail_f16_4100", M=4100, N=4104, K=4096, seed=7370),
    CFG[3].replace(name="tail_i8_mmajorA_cdm", M=4112, N=4100, K=8192, L=1, cd_major="M", seed=7380),
    CFG[1].replace(name="tail_bf16_f32_l2", M=2100, N=3848, K=4096, L=2, seed=7390),
]


@pytest.mark.parametrize("p", SPLIT_TAIL, ids=[e.name for e in SPLIT_TAIL])
def test_parity_split_last_round(p):
    _say("case", p.name, p.M, p.N, p.K, p.L, p.cd_major)
    (ed, ey), plan, npts = parity_sampled(p, sub=32)
    cus = plan["cus"]
    tail = plan["tiles"] % cus
    ktiles = -(-p.K // plan["tile_k"])
    s = plan["splits"]
    assert plan["tiles"] > cus and 0 < tail <= cus // 2, plan
    assert plan["split_tiles"] == tail and 2 <= s <= min(cus // tail, ktiles // 4, 16), plan
    assert plan["grid"] == cus
    assert plan["workspace_bytes"] == s * tail * plan["tile_m"] * plan["tile_n"] * 4
    _say("  plan", plan["name"], "split tiles", tail, "splits", s, "points", npts,
         "err D %.3g Y %.3g" % (ed, ey))


def test_create_refuses_more_than_2_31_work_items():
    """Tile and work-item numbers are 32-bit in the kernels: a plan of 2^31
    or more work items is refused at create (no tensor is allocated)."""
    import beta_epilogue_amd as ge
    with pytest.raises(ge.GemmEpiError) as e:
        ge.FusedGemm(1 << 19, 1 << 19, 64, 600, ab="f16", d="f16")
    assert e.value.code == ge.GEMM_EPI_ERR_UNSUPPORTED and "work items" in str(e.value), str(e.value)


def test_split_not_chosen_for_a_short_last_round():
    """The same last round with K = 512: slicing saves less than the
    reduction kernel costs, so every tile runs whole."""
    import beta_epilogue_amd as ge
    g = ge.FusedGemm(4100, 4104, 512, ab="f16", c="f16", x="f16", d="f16", y="f16")
    assert g.plan["splits"] == 1 and g.plan["split_tiles"] == 0 and g.plan["workspace_bytes"] == 0
    g.close()


# uint8 A/B (int32 accumulation): the int8 MFMA on the bytes with their top
# bit flipped, plus the sums of the unsigned rows and columns along K in the
# epilogue.  Bit-exact against the oracle in every layout.
U8 = [
    CFG[3].replace(name="u8_kk_n", M=272, N=264, K=400, L=2, a_major="K", ab="u8",
                   dist_ab="u8full", seed=7500),
    CFG[3].replace(name="u8_mk_n_xy", M=272, N=264, K=4096, L=1, ab="u8", dist_ab="u8full",
                   x="i32", y="i32", alpha=-3.0, beta=2.0, x_factor=5.0, dist_x="i1000",
                   seed=7510),
    CFG[3].replace(name="u8_kn_m", M=260, N=272, K=144, L=2, a_major="K", b_major="N",
                   cd_major="M", ab="u8", dist_ab="u8full", seed=7520),
    CFG[3].replace(name="u8_mn_m_relu", M=288, N=272, K=48, L=3, b_major="N", cd_major="M",
                   ab="u8", dist_ab="u8full", beta=-1.0, epilogue="relu", seed=7530),
    CFG[3].replace(name="u8_tiny", M=16, N=16, K=16, L=2, ab="u8", dist_ab="u8full", seed=7540),
]


@pytest.mark.parametrize("p", U8, ids=[e.name for e in U8])
def test_parity_u8(p):
    _say("case", p.name, p.M, p.N, p.K, p.L, p.a_major, p.b_major, p.cd_major)
    (ed, ey), plan = parity_full(p)
    # the sums of A rows and B columns, then the flipped copies of A and B,
    # each part at a 256-byte boundary
    up = lambda x: (x + 255) // 256 * 256
    ws = up(p.L * (p.M + p.N) * 4) + up(p.L * p.M * p.K) + up(p.L * p.N * p.K)
    assert plan["splits"] == 1 and plan["workspace_bytes"] == ws
    _say("  plan", plan["name"])


def test_parity_u8_full_size_sampled():
    """The batched int8 workload's shape (4096^3 x 4, A M-major) in uint8."""
    p = CFG[3].replace(name="u8_4096x4_mmajorA", ab="u8", dist_ab="u8full", seed=7550)
    _say("case", p.name)
    (ed, ey), plan, npts = parity_sampled(p)
    _say("  plan", plan["name"], "points", npts)


def test_beta_zero_does_not_read_c():
    """beta = 0 skips C: NaN in C cannot reach D (C is given but unread)."""
    p = CFG[2].replace(name="beta0_nan_c", M=256, N=264, K=64, beta=0.0, x_factor=0.0)
    ins = synth.make_inputs(p)
    ins["C"] = torch.full_like(ins["C"], float("nan"))
    ins["X"] = torch.full_like(ins["X"], float("nan"))
    _say("case", p.name)
    D, Y, _ = run_gpu(p, ins)
    assert np.all(np.isfinite(to_f64(D)))
    (ed, ey), _ = parity_full(p, ins=ins)


def test_every_variant_runs():
    """Each compiled kernel variant passes parity on a problem it accepts (its
    A/B type, A, B and C/D majorness; ragged M, N, K; two batches)."""
    import beta_epilogue_amd as ge
    names = [ge.gemm_epi_variant_name(i) for i in range(ge.gemm_epi_variant_count())]
    base = {
        "f16": CFG[2].replace(M=264, N=272, K=136, L=2),
        "bf16": CFG[1].replace(M=264, N=272, K=136, L=2),
        "e4m3": CFG[4].replace(M=272, N=288, K=144, L=2),
        "e5m2": CFG[4].replace(M=272, N=288, K=144, L=2, ab="e5m2", dist_ab="e5m2tab"),
        "e4e5": CFG[4].replace(M=272, N=288, K=144, L=2, b_ab="e5m2", dist_b="e5m2tab"),
        "e5e4": CFG[4].replace(M=272, N=288, K=144, L=2, ab="e5m2", dist_ab="e5m2tab",
                               b_ab="e4m3", dist_b="e4m3tab"),
        "i8": CFG[3].replace(M=272, N=288, K=144, L=2),
        "u8": CFG[3].replace(M=272, N=288, K=144, L=2, ab="u8", dist_ab="u8full"),
    }
    for i, name in enumerate(names):
        ab, layout, cd = name.split("_")[0:3]
        p = base[ab].replace(name="variant_" + name,
                             a_major="K" if layout[0] == "k" else "M",
                             b_major="K" if layout[1] == "k" else "N",
                             cd_major=cd.upper())
        _say("variant", i, name)
        (ed, ey), plan = parity_full(p, variant=i)
        assert plan["name"] == name


def test_ring_depth_k_extents():
    """Each multi-stage variant at K extents with fewer, as many and more K
    tiles than ring stages, and a ragged K tail (the prologue, the counted
    waits and the refill of a stage in the step after its barrier)."""
    import beta_epilogue_amd as ge
    names = [ge.gemm_epi_variant_name(i) for i in range(ge.gemm_epi_variant_count())]
    for i, name in enumerate(names):
        parts = name.split("_")
        if not name.startswith("f16_kk") or not any(q.startswith("s") and q[1:].isdigit()
                                                   and int(q[1:]) >= 3 for q in parts):
            continue
        for K in (8, 40, 72, 136, 168, 200, 520):
            p = CFG[2].replace(name="ring_%s_K%d" % (name, K), M=264, N=272, K=K, L=1)
            _say("variant", i, name, "K", K)
            (ed, ey), plan = parity_full(p, variant=i)
            assert plan["name"] == name


def test_run_rejects_misaligned_pointer():
    import beta_epilogue_amd as ge
    p = CFG[2].replace(M=64, N=64, K=64)
    g = ge.FusedGemm(p.M, p.N, p.K, ab="f16", c="f16", x="f16", d="f16", y="f16")
    a = torch.zeros(64 * 64 + 8, dtype=torch.float16, device="cuda")
    d = torch.zeros(64 * 64, dtype=torch.float16, device="cuda")
    y = torch.zeros(64 * 64, dtype=torch.float16, device="cuda")
    with pytest.raises(ge.GemmEpiError) as e:
        ge.gemm_epi_run(g.handle, a.data_ptr() + 2, a.data_ptr(), None, None,
                        d.data_ptr(), y.data_ptr(), 1.0, 0.0, 0.0, None)
    assert e.value.code == ge.GEMM_EPI_ERR_ALIGNMENT
    with pytest.raises(ge.GemmEpiError) as e:  # Y required: y_dtype is set
        ge.gemm_epi_run(g.handle, a.data_ptr(), a.data_ptr(), None, None,
                        d.data_ptr(), None, 1.0, 0.0, 0.0, None)
    assert e.value.code == ge.GEMM_EPI_ERR_INVALID_ARG
    g.close()


def test_int_scalars_must_be_integral():
    import beta_epilogue_amd as ge
    g = ge.FusedGemm(64, 64, 64, ab="i8", c="i32", d="i32")
    a = torch.zeros(64 * 64, dtype=torch.int8, device="cuda")
    d = torch.zeros(64 * 64, dtype=torch.int32, device="cuda")
    with pytest.raises(ge.GemmEpiError) as e:
        g(a, a, d, D=d, alpha=1.5, beta=1.0)
    assert e.value.code == ge.GEMM_EPI_ERR_UNSUPPORTED
    g.close()


def _random_problem(i):
    """Seeded random problem i: A/B type (fp8 pairs included), layouts,
    ragged M, N, K within the 16-byte rule, batch, output types, scalars and
    epilogue form."""
    rng = np.random.default_rng(9000 + i)
    kind = ["f16", "bf16", "e4m3", "e5m2", "i8", "e4e5", "e5e4"][i % 7]
    ab, b_ab = {"e4e5": ("e4m3", "e5m2"), "e5e4": ("e5m2", "e4m3")}.get(kind, (kind, None))
    dist = {"f16": "normal", "bf16": "normal", "e4m3": "e4m3tab", "e5m2": "e5m2tab",
            "i8": "i8full"}
    cd = "NM"[int(rng.integers(2))]
    a_major = "KM"[int(rng.integers(2))]
    b_major = "KN"[int(rng.integers(2))]
    kq = 8 if ab in ("f16", "bf16") else 16
    K = int(kq * rng.integers(1, 40))
    L = int(rng.integers(1, 4))
    if ab == "i8":
        outs = ["i32"]
    else:
        outs = ["f32", "f16", "bf16"]
    d = outs[int(rng.integers(len(outs)))]
    c = outs[int(rng.integers(len(outs)))] if rng.integers(3) else None
    x = outs[int(rng.integers(len(outs)))] if rng.integers(2) else None
    y = outs[int(rng.integers(len(outs)))] if rng.integers(2) else None
    # contiguous C/D extent: a multiple of 8 elements covers every output type
    cdq = 8
    M = int(rng.integers(1, 600))
    N = int(rng.integers(1, 600))
    if cd == "N":
        N = max(cdq, N // cdq * cdq)
    else:
        M = max(cdq, M // cdq * cdq)
    if a_major == "M":  # the 16-byte rule on M-major A / N-major B
        M = max(16, M // 16 * 16)
    if b_major == "N":
        N = max(16, N // 16 * 16)
    if ab == "i8":
        alpha, beta, xf = (float(rng.integers(-3, 4)) for _ in range(3))
    else:
        alpha, beta, xf = (float(np.round(rng.uniform(-2, 2), 3)) for _ in range(3))
    return synth.Problem(
        "random_%d_%s_%s%s%s_%s" % (i, kind, a_major.lower(), b_major.lower(), cd.lower(), d),
        M, N, K, L, ab, a_major=a_major, b_major=b_major, cd_major=cd, c=c, x=x, d=d, y=y, alpha=alpha,
        beta=beta if c else 0.0, x_factor=xf if x else 0.0, dist_ab=dist[ab],
        dist_c="i1000" if ab == "i8" else "normal", dist_x="i1000" if ab == "i8" else "normal",
        seed=9100 + 10 * i, epilogue="relu" if rng.integers(2) else "linear", b_ab=b_ab,
        dist_b=dist[b_ab] if b_ab else None)


RANDOM = [_random_problem(i) for i in range(64)]


@pytest.mark.parametrize("p", RANDOM, ids=[r.name for r in RANDOM])
def test_parity_random_problems(p):
    """Seeded random shapes, layouts, types and scalars against the oracle."""
    _say("case", p.name, p.M, p.N, p.K, p.L, p.c, p.x, p.d, p.y, p.epilogue)
    (ed, ey), plan = parity_full(p)
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


def _random_typed(i):
    """Problem i with one output type for every C/X/D/Y in use (the typed
    epilogue, which the 16x16-block defaults run), or None for fp8 inputs."""
    p = _random_problem(i)
    if p.ab not in ("f16", "bf16", "i8"):
        return None
    t = p.d
    return p.replace(name=p.name + "_typed", c=t if p.c else None, x=t if p.x else None,
                     y=t if p.y else None)


RANDOM_TYPED = [q for q in (_random_typed(i) for i in range(200, 290)) if q is not None]


@pytest.mark.parametrize("p", RANDOM_TYPED, ids=[r.name for r in RANDOM_TYPED])
def test_parity_random_typed(p):
    """Seeded random problems through the one-type epilogue."""
    _say("case", p.name, p.M, p.N, p.K, p.L, p.d, p.epilogue)
    (ed, ey), plan = parity_full(p)
    _say("  plan", plan["name"], "err D %.3g Y %.3g" % (ed, ey))


"""Shared GPU-parity helpers: run the HIP library through its C ABI and
compare with the CPU oracle on the same seeded inputs.

Bars (per the operation's error analysis; the pages fix no tolerance):
  * int32 outputs (int8 inputs): bit-exact;
  * problems whose every intermediate is exactly representable (integer
    inputs, dyadic scalars): bit-exact, in the spirit of the CuTe tutorial's
    "relative error <= 0" check;
  * float outputs: per element
        |D - D_ref| / (|alpha| S + |beta C| + |x_factor X|) <= tol,
        |Y - Y_ref| / S <= tol,
    S = sum_k |a||b|, tol = 1e-5 for fp32 and 1e-3 for fp16 outputs
    (bf16 outputs: 2^-8, since bf16's own rounding step is 2^-9 relative),
    set by the output type alone; a zero denominator demands equality.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
import beta_epilogue_amd as ge

GUARD = 64  # elements of guard band before and after every output
SENTINEL = {"f16": -12345.0, "bf16": -12345.0, "f32": -12345.0,
            "i32": 0x5A5A5A5A}


def tolerance(dtype: str) -> float:
    """Normalised-error bar for an output type, whatever the input types:
    1e-5 for fp32, 1e-3 for fp16 and 2^-8 for bf16 outputs (bf16's own
    rounding step, 2^-9 relative, exceeds 1e-3)."""
    return {"f32": 1e-5, "f16": 1e-3, "bf16": 2.0 ** -8}[dtype]


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Library decode of stored values (torch's conversion) to float64."""
    t = t.detach().cpu().reshape(-1)
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        t = t.to(torch.float32)
    return t.to(torch.float64).numpy()


class GuardedOut:
    """An output tensor with sentinel-filled guard bands on both sides."""

    def __init__(self, dtype: str, shape, device="cuda"):
        n = int(np.prod(shape))
        td = synth.TORCH_DTYPE[dtype]
        self.buf = torch.full((n + 2 * GUARD,), SENTINEL[dtype], dtype=td,
                              device=device)
        self.t = self.buf[GUARD:GUARD + n].view(shape)
        self.dtype = dtype

    def guards_intact(self) -> bool:
        s = SENTINEL[self.dtype]
        lo, hi = self.buf[:GUARD], self.buf[-GUARD:]
        return bool(torch.all(lo == s).item()) and bool(torch.all(hi == s).item())


def run_gpu(p: synth.Problem, ins, variant=-1, check_inputs=True, splits=0, static_scratch=False):
    """Run problem p on the GPU through the C ABI.  Returns host D, Y.
    splits: the K split asked for (0: the library's choice);
    static_scratch: run through gemm_epi_run_static."""
    dev = {k: (v.cuda() if v is not None else None) for k, v in ins.items()}
    keep = {k: v.clone() for k, v in dev.items() if v is not None and k in "CX"}
    g = ge.FusedGemm(p.M, p.N, p.K, p.L, ab=p.ab, a_major=p.a_major,
                     b_major=p.b_major, cd_major=p.cd_major, c=p.c, x=p.x,
                     d=p.d, y=p.y, variant=variant, epilogue=p.epilogue, b=p.b_ab,
                     splits=splits)
    shape = p.storage_shape("D")
    D = GuardedOut(p.d, shape)
    Y = GuardedOut(p.y, shape) if p.y else None
    g(dev["A"], dev["B"], dev["C"], dev["X"], D=D.t, Y=Y.t if Y else None,
      alpha=p.alpha, beta=p.beta, x_factor=p.x_factor, static_scratch=static_scratch)
    torch.cuda.synchronize()
    assert D.guards_intact(), "D guard band overwritten"
    if Y:
        assert Y.guards_intact(), "Y guard band overwritten"
    if check_inputs:
        for k, v in keep.items():  # bytes compare: NaN inputs must stay NaN
            assert torch.equal(v.reshape(-1).view(torch.uint8),
                               dev[k].reshape(-1).view(torch.uint8)), "%s was modified" % k
    plan = g.plan
    g.close()
    return D.t.cpu(), (Y.t.cpu() if Y else None), plan


def _den(p, S, cvals, xvals):
    den = abs(p.alpha) * S
    if cvals is not None and p.beta != 0.0:
        den = den + np.abs(p.beta * cvals)
    if xvals is not None and p.x_factor != 0.0:
        den = den + np.abs(p.x_factor * xvals)
    return den


def check(p: synth.Problem, D_gpu, Y_gpu, Dref, Yref, S, cvals, xvals,
          exact=False):
    """Compare GPU outputs (flat, any order) with oracle values at the same
    positions.  Returns (max err D, max err Y)."""
    d = to_f64(D_gpu)
    if p.d == "i32" or exact:
        if p.d == "i32":
            assert np.all(np.abs(Dref) < 2.0 ** 31), "reference outside int32"
        bad = np.nonzero(d != Dref)[0]
        assert bad.size == 0, "D not exact at %d places, first %s: got %r want %r" % (
            bad.size, bad[:5], d[bad[:5]], Dref[bad[:5]])
        errd = 0.0
    else:
        den = _den(p, S, cvals, xvals)
        diff = np.abs(d - Dref)
        zero = den == 0
        assert np.all(diff[zero] == 0), "D differs where the bound is 0"
        err = np.where(zero, 0.0, diff / np.where(zero, 1.0, den))
        errd = float(err.max()) if err.size else 0.0
        tol = tolerance(p.d)
        assert errd <= tol, "D normalised error %.3g > %.3g at %s" % (
            errd, tol, np.argmax(err))
    erry = 0.0
    if p.y:
        y = to_f64(Y_gpu)
        if p.y == "i32" or exact:
            assert np.array_equal(y, Yref), "Y not exact"
        else:
            diff = np.abs(y - Yref)
            zero = S == 0
            assert np.all(diff[zero] == 0)
            err = np.where(zero, 0.0, diff / np.where(zero, 1.0, S))
            erry = float(err.max()) if err.size else 0.0
            assert erry <= tolerance(p.y), "Y normalised error %.3g" % erry
    return errd, erry


def parity_full(p: synth.Problem, variant=-1, exact=False, ins=None, splits=0):
    """Whole-output parity against the full oracle result."""
    ins = ins if ins is not None else synth.make_inputs(p)
    D, Y, plan = run_gpu(p, ins, variant, splits=splits)
    Dref, Yref, S = oracle.gemm_epi(p.M, p.N, p.K, p.L, ins["A"], ins["B"],
                                    ins["C"], ins["X"], ab=p.ab, b=p.b_ab, c=p.c, x=p.x,
                                    a_major=p.a_major, b_major=p.b_major,
                                    cd_major=p.cd_major, alpha=p.alpha,
                                    beta=p.beta, x_factor=p.x_factor,
                                    relu=p.epilogue == "relu")
    cv = to_f64(ins["C"]) if ins["C"] is not None else None
    xv = to_f64(ins["X"]) if ins["X"] is not None else None
    errs = check(p, D.reshape(-1), Y.reshape(-1) if Y is not None else None,
                 Dref, Yref, S, cv, xv, exact=exact)
    return errs, plan


def sample_points(p: synth.Problem, n_random=2048, seed=7, tile=256, sub=128):
    """Whole rows and columns at the edges and middle, one random point in
    every sub x sub quadrant of every tile x tile output tile of every batch
    (so a tile the persistent schedule dropped, duplicated or misplaced, or a
    wave that wrote another wave's quadrant, fails), plus random points."""
    rng = np.random.default_rng(seed)
    pts = []
    for l in sorted({0, p.L - 1}):
        for m in sorted({0, p.M - 1, (p.M // 2 + 3) % p.M}):
            pts += [(l, m, n) for n in range(p.N)]
        for n in sorted({0, p.N - 1, (p.N // 3 + 5) % p.N}):
            pts += [(l, m, n) for m in range(p.M)]
    m0 = np.arange(0, p.M, sub)
    n0 = np.arange(0, p.N, sub)
    ll, mm, nn = np.meshgrid(np.arange(p.L), m0, n0, indexing="ij")
    ll, mm, nn = ll.reshape(-1), mm.reshape(-1), nn.reshape(-1)
    mq = mm + (rng.random(mm.size) * np.minimum(sub, p.M - mm)).astype(np.int64)
    nq = nn + (rng.random(nn.size) * np.minimum(sub, p.N - nn)).astype(np.int64)
    quad = np.stack([ll, mq, nq], axis=1)
    r = np.stack([rng.integers(0, p.L, n_random), rng.integers(0, p.M, n_random),
                  rng.integers(0, p.N, n_random)], axis=1)
    pts = np.concatenate([np.asarray(pts, np.int64).reshape(-1, 3), quad, r])
    return np.unique(pts, axis=0)


def flat_index(p: synth.Problem, pts):
    l, m, n = pts[:, 0], pts[:, 1], pts[:, 2]
    if p.cd_major == "N":
        return l * p.M * p.N + m * p.N + n
    return l * p.M * p.N + n * p.M + m


def parity_sampled(p: synth.Problem, variant=-1, n_random=2048, ins=None, sub=128):
    """Full-size run, compared at sampled outputs the oracle computes one by
    one (edge and middle rows/columns, a point in every sub x sub block of
    every output tile, random points)."""
    ins = ins if ins is not None else synth.make_inputs(p)
    D, Y, plan = run_gpu(p, ins, variant)
    pts = sample_points(p, n_random, sub=sub)
    Dref, Yref, S = oracle.gemm_epi_points(
        p.M, p.N, p.K, p.L, ins["A"], ins["B"], ins["C"], ins["X"], points=pts,
        ab=p.ab, b=p.b_ab, c=p.c, x=p.x, a_major=p.a_major, b_major=p.b_major,
        cd_major=p.cd_major, alpha=p.alpha, beta=p.beta, x_factor=p.x_factor,
        relu=p.epilogue == "relu")
    idx = flat_index(p, pts)
    cv = to_f64(ins["C"])[idx] if ins["C"] is not None else None
    xv = to_f64(ins["X"])[idx] if ins["X"] is not None else None
    Ds = D.reshape(-1)[torch.from_numpy(idx)]
    Ys = Y.reshape(-1)[torch.from_numpy(idx)] if Y is not None else None
    errs = check(p, Ds, Ys, Dref, Yref, S, cv, xv)
    return errs, plan, len(pts)

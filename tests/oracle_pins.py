"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError if the
oracle disagrees with something fixed independently of its code: the number
formats' definitions (golden codes), a library decoder, exact rational brute
force, closed forms of the operation, an independent fp64 library matmul, or
an invariant of the definition (majorness duality, batch independence,
linearity, the skip rule for absent terms).

The operation pinned is the one the CuTe DSL example
``custom_epilogue_dense_gemm.py`` documents in its module docstring
("Tensor dimensions" and the epilogue formula): Y = A.B^T per batch and
D = alpha*Y + beta*C + x_factor*X, and the clamped form its epilogue function
builds, D = max(0, alpha*Y + beta*C) + x_factor*X.  The same pins are run against copies of
the oracle with planted mistakes (see test_oracle_mutants.py), each of which
must fail at least one of them.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "number_formats.txt")

FLOAT_AB = ("f16", "bf16", "e4m3", "e5m2")
INT_AB = ("i8", "u8")
ALL_AB = FLOAT_AB + INT_AB
LAYOUTS = [(a, b, cd) for a in "KM" for b in "KN" for cd in "NM"]


# --------------------------------------------------------------------------
# helpers (independent of the oracle's C code)
# --------------------------------------------------------------------------

def lib_decode(t: torch.Tensor) -> np.ndarray:
    """Library decode: torch's own conversion of the stored type to float64."""
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2):
        return t.to(torch.float32).to(torch.float64).reshape(-1).numpy()
    return t.to(torch.float64).reshape(-1).numpy()


def logical(stored: torch.Tensor, which: str, major: str) -> torch.Tensor:
    """(L, rows, K) or (L, M, N) logical view of a packed stored operand."""
    if which in "AB":
        return stored if major == "K" else stored.transpose(1, 2)
    return stored if major == "N" else stored.transpose(1, 2)


def store(logical_t: torch.Tensor, which: str, major: str) -> torch.Tensor:
    """Packed storage of a logical (L, rows, cols) tensor in ``major``."""
    if which in "AB":
        s = logical_t if major == "K" else logical_t.transpose(1, 2)
    else:
        s = logical_t if major == "N" else logical_t.transpose(1, 2)
    return s.contiguous()


def to_cd_layout(t_lmn: np.ndarray, cd: str) -> np.ndarray:
    """Flatten an (L, M, N) array into the C/D storage order."""
    return (t_lmn if cd == "N" else np.swapaxes(t_lmn, 1, 2)).reshape(-1)


def from_cd_layout(flat: np.ndarray, L, M, N, cd: str) -> np.ndarray:
    if cd == "N":
        return flat.reshape(L, M, N)
    return np.swapaxes(flat.reshape(L, N, M), 1, 2)


def run(orc, A, B, C=None, X=None, *, M, N, K, L, ab, c=None, x=None,
        a="K", b="K", cd="N", alpha=1.0, beta=0.0, xf=0.0, relu=False, bt=None):
    D, Y, S = orc.gemm_epi(M, N, K, L, A, B, C, X, ab=ab, b=bt, c=c, x=x,
                           a_major=a, b_major=b, cd_major=cd, alpha=alpha,
                           beta=beta, x_factor=xf, relu=relu, nthreads=2)
    return (from_cd_layout(D, L, M, N, cd), from_cd_layout(Y, L, M, N, cd),
            from_cd_layout(S, L, M, N, cd))


def _parse_value(tok: str):
    if tok in ("inf", "-inf", "nan"):
        return float(tok)
    if tok == "-0":
        return -0.0
    if "*2^" in tok:
        p, e = tok.split("*2^")
        return math.ldexp(int(p), int(e))
    if "/" in tok:
        p, q = tok.split("/")
        return int(p) / int(q)  # exact: q is a power of two here
    return float(int(tok))


def _rand(dist, dtype, shape, seed):
    n = int(np.prod(shape))
    return synth.draw(dist, dtype, n, seed).view(shape)


def _dist_for(ab):
    return {"f16": "normal", "bf16": "normal", "e4m3": "e4m3tab", "e5m2": "e5m2tab",
            "i8": "i8full", "u8": "u8full"}[ab]


# --------------------------------------------------------------------------
# decoding pins
# --------------------------------------------------------------------------

def pin_decode_golden(orc):
    """Stored codes with values fixed by the formats' definitions."""
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            typ, code, val = line.split()[:3]
            code = int(code, 16)
            arr = np.array([code], dtype=np.uint8 if typ in ("e4m3", "e5m2") else np.uint16)
            got = orc.decode(typ, arr)[0]
            want = _parse_value(val)
            if math.isnan(want):
                assert math.isnan(got), (typ, hex(code), got)
            else:
                assert got == want and math.copysign(1, got) == math.copysign(1, want), \
                    (typ, hex(code), got, want)


def pin_decode_vs_library(orc):
    """Every f16, bf16 and e4m3 code decodes as torch decodes it."""
    codes16 = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    for typ, td in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        got = orc.decode(typ, codes16.numpy().view(np.uint16))
        want = lib_decode(codes16.view(td))
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), typ
        assert np.array_equal(got[~nan], want[~nan]), typ
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), typ
    codes8 = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for typ, td in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        got = orc.decode(typ, codes8.numpy())
        want = lib_decode(codes8.view(td))
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), typ
        assert np.array_equal(got[~nan], want[~nan]), typ
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), typ
    i8 = np.arange(-128, 128, dtype=np.int8)
    assert np.array_equal(orc.decode("i8", i8), i8.astype(np.float64))
    u8 = np.arange(256, dtype=np.uint8)  # every code is its unsigned value
    assert np.array_equal(orc.decode("u8", u8), np.arange(256, dtype=np.float64))
    i32 = np.array([0, 1, -1, 2**31 - 1, -2**31, 123456789], dtype=np.int32)
    assert np.array_equal(orc.decode("i32", i32), i32.astype(np.float64))
    f32 = np.array([0.0, -1.5, 3.4028234663852886e38, 1e-45, 0.1], np.float32)
    assert np.array_equal(orc.decode("f32", f32), f32.astype(np.float64))


# --------------------------------------------------------------------------
# contraction + epilogue pins
# --------------------------------------------------------------------------

def pin_bruteforce_exact(orc):
    """Tiny problems, every input type and layout: the oracle equals exact
    rational arithmetic to within the fp64 rounding bound (exactly, for
    integer inputs)."""
    M, N, K, L = 3, 4, 5, 2
    seed = 90000
    for ab in ALL_AB:
        for (a, b, cd) in LAYOUTS:
            seed += 10
            Al = _rand(_dist_for(ab), ab, (L, M, K), seed + 1)
            Bl = _rand(_dist_for(ab), ab, (L, N, K), seed + 2)
            if ab in INT_AB:
                c, x = "i32", "i32"
                Cl = _rand("i1000", "i32", (L, M, N), seed + 3)
                Xl = _rand("i1000", "i32", (L, M, N), seed + 4)
                alpha, beta, xf = 3.0, -2.0, 5.0
            else:
                c, x = {"f16": ("f32", "f16"), "bf16": ("bf16", "f32"),
                        "e4m3": ("f16", "bf16"), "e5m2": ("bf16", "f16")}[ab]
                Cl = _rand("normal", c, (L, M, N), seed + 3)
                Xl = _rand("normal", x, (L, M, N), seed + 4)
                alpha, beta, xf = 1.75, -0.625, 2.5
            D, Y, S = run(orc, store(Al, "A", a), store(Bl, "B", b),
                          store(Cl, "C", cd), store(Xl, "X", cd), M=M, N=N,
                          K=K, L=L, ab=ab, c=c, x=x, a=a, b=b, cd=cd,
                          alpha=alpha, beta=beta, xf=xf)
            av = lib_decode(Al).reshape(L, M, K)
            bv = lib_decode(Bl).reshape(L, N, K)
            cv = lib_decode(Cl).reshape(L, M, N)
            xv = lib_decode(Xl).reshape(L, M, N)
            for l in range(L):
                for m in range(M):
                    for n in range(N):
                        acc = sum(Fraction(av[l, m, k]) * Fraction(bv[l, n, k])
                                  for k in range(K))
                        s = sum(abs(Fraction(av[l, m, k]) * Fraction(bv[l, n, k]))
                                for k in range(K))
                        d = (Fraction(alpha) * acc + Fraction(beta) * Fraction(cv[l, m, n])
                             + Fraction(xf) * Fraction(xv[l, m, n]))
                        if ab in INT_AB:
                            assert Y[l, m, n] == acc and D[l, m, n] == d and S[l, m, n] == s, \
                                (ab, a, b, cd, l, m, n)
                        else:
                            den = (abs(alpha) * s + abs(Fraction(beta) * Fraction(cv[l, m, n]))
                                   + abs(Fraction(xf) * Fraction(xv[l, m, n])))
                            bound = float(den) * (K + 4) * 2.0 ** -52
                            assert abs(Fraction(Y[l, m, n]) - acc) <= Fraction(float(s) * (K + 1) * 2.0 ** -52), \
                                (ab, a, b, cd, "Y", l, m, n)
                            assert abs(Fraction(D[l, m, n]) - d) <= Fraction(bound), \
                                (ab, a, b, cd, "D", l, m, n)
                            assert abs(Fraction(S[l, m, n]) - s) <= Fraction(float(s) * (K + 1) * 2.0 ** -52)


def pin_identity_A(orc):
    """A = I (M = K): D[m, n] = alpha*B[n, m] + beta*C[m, n], exactly."""
    M = K = 6
    N, L = 5, 2
    for ab in ALL_AB:
        for a in "KM":
            eye = torch.eye(M, dtype=torch.float32).expand(L, M, M).to(
                synth.TORCH_DTYPE[ab])
            Bl = _rand(_dist_for(ab), ab, (L, N, K), 777)
            if ab in INT_AB:
                c, alpha, beta = "i32", 3.0, -2.0
                Cl = _rand("i1000", "i32", (L, M, N), 778)
            else:
                c, alpha, beta = "f32", 0.5, 2.0
                Cl = _rand("normal", "f32", (L, M, N), 778)
            D, Y, _ = run(orc, store(eye, "A", a), store(Bl, "B", "K"), Cl,
                          M=M, N=N, K=K, L=L, ab=ab, c=c, a=a, alpha=alpha,
                          beta=beta)
            bv = lib_decode(Bl).reshape(L, N, K)
            cv = lib_decode(Cl).reshape(L, M, N)
            want_y = np.swapaxes(bv, 1, 2)
            assert np.array_equal(Y, want_y), (ab, a)
            assert np.array_equal(D, alpha * want_y + beta * cv), (ab, a)


def pin_identity_B(orc):
    """B = I (N = K): D = alpha*A + beta*C, exactly."""
    N = K = 7
    M, L = 4, 1
    for ab in ALL_AB:
        for b in "KN":
            eye = torch.eye(N, dtype=torch.float32).expand(L, N, N).to(
                synth.TORCH_DTYPE[ab])
            Al = _rand(_dist_for(ab), ab, (L, M, K), 555)
            c = "i32" if ab in INT_AB else "f16"
            Cl = _rand("i1000" if ab in INT_AB else "normal", c, (L, M, N), 556)
            D, Y, _ = run(orc, store(Al, "A", "K"), store(eye, "B", b), Cl,
                          M=M, N=N, K=K, L=L, ab=ab, c=c, b=b, alpha=-2.0,
                          beta=0.25 if ab not in INT_AB else 4.0)
            av = lib_decode(Al).reshape(L, M, K)
            cv = lib_decode(Cl).reshape(L, M, N)
            beta = 0.25 if ab not in INT_AB else 4.0
            assert np.array_equal(Y, av), (ab, b)
            assert np.array_equal(D, -2.0 * av + beta * cv), (ab, b)


def pin_all_ones(orc):
    """A, B all ones: every Y is K and every S is K."""
    M, N, K, L = 3, 5, 37, 2
    for ab in ALL_AB:
        one = torch.ones(L, M, K).to(synth.TORCH_DTYPE[ab])
        oneb = torch.ones(L, N, K).to(synth.TORCH_DTYPE[ab])
        D, Y, S = run(orc, one, oneb, M=M, N=N, K=K, L=L, ab=ab, alpha=2.0)
        assert np.all(Y == K) and np.all(S == K) and np.all(D == 2 * K), ab


def pin_rank1(orc):
    """A[m,k] = u_m p_k and B[n,k] = w_n q_k give Y = (p.q) u_m w_n.  u and w
    are powers of two, so every product is exact in each input format (e5m2
    has two fraction bits)."""
    M, N, K, L = 4, 6, 9, 1
    u = torch.tensor([1.0, -2.0, 0.5, 4.0])
    w = torch.tensor([2.0, 1.0, -1.0, 0.25, -4.0, 0.5])
    p = torch.tensor([1.0, -1.0, 2.0, 0.5, -0.5, 3.0, 1.0, -2.0, 0.25])
    q = torch.tensor([0.5, 2.0, -1.0, 1.0, 4.0, -0.25, 1.0, 0.5, -3.0])
    pq = float((p.double() * q.double()).sum())
    for ab in FLOAT_AB:
        for a in "KM":
            for b in "KN":
                A = (u[:, None] * p[None, :]).expand(L, M, K).to(synth.TORCH_DTYPE[ab])
                B = (w[:, None] * q[None, :]).expand(L, N, K).to(synth.TORCH_DTYPE[ab])
                D, Y, _ = run(orc, store(A, "A", a), store(B, "B", b), M=M,
                              N=N, K=K, L=L, ab=ab, a=a, b=b)
                want = pq * np.outer(u.double().numpy(), w.double().numpy())
                assert np.array_equal(Y[0], want), (ab, a, b)


def pin_alpha_zero(orc):
    """alpha = 0: D = beta*C + x_factor*X exactly, whatever A and B are."""
    M, N, K, L = 5, 3, 8, 2
    for cd in "NM":
        Al = _rand("normal", "f16", (L, M, K), 11)
        Bl = _rand("normal", "f16", (L, N, K), 12)
        Cl = _rand("normal", "f16", (L, M, N), 13)
        Xl = _rand("normal", "bf16", (L, M, N), 14)
        D, _, _ = run(orc, Al, Bl, store(Cl, "C", cd), store(Xl, "X", cd),
                      M=M, N=N, K=K, L=L, ab="f16", c="f16", x="bf16", cd=cd,
                      alpha=0.0, beta=1.5, xf=-3.0)
        want = 1.5 * lib_decode(Cl).reshape(L, M, N) - 3.0 * lib_decode(Xl).reshape(L, M, N)
        assert np.array_equal(D, want), cd


def pin_skip_and_identity_epilogue(orc):
    """alpha = 1, beta = x_factor = 0: D equals Y bit for bit, and C, X
    (full of NaN) are not read."""
    M, N, K, L = 4, 4, 16, 1
    Al = _rand("normal", "bf16", (L, M, K), 21)
    Bl = _rand("normal", "bf16", (L, N, K), 22)
    nan = torch.full((L, M, N), float("nan"), dtype=torch.float32)
    D, Y, _ = run(orc, Al, Bl, nan, nan.clone(), M=M, N=N, K=K, L=L, ab="bf16",
                  c="f32", x="f32", alpha=1.0, beta=0.0, xf=0.0)
    assert np.array_equal(D, Y) and np.all(np.isfinite(D))
    # and a present, non-zero beta does read C
    D2, _, _ = run(orc, Al, Bl, nan, None, M=M, N=N, K=K, L=L, ab="bf16",
                   c="f32", alpha=1.0, beta=1.0)
    assert np.all(np.isnan(D2))


def pin_integer_exact(orc):
    """int8, uint8 and integer-valued fp16: Y equals numpy's int64 matmul."""
    M, N, K, L = 9, 7, 300, 2
    Al = _rand("i8full", "i8", (L, M, K), 31)
    Bl = _rand("i8full", "i8", (L, N, K), 32)
    Cl = _rand("i1000", "i32", (L, M, N), 33)
    for a in "KM":
        for cd in "NM":
            D, Y, S = run(orc, store(Al, "A", a), Bl, store(Cl, "C", cd),
                          M=M, N=N, K=K, L=L, ab="i8", c="i32", a=a, cd=cd,
                          alpha=1.0, beta=1.0)
            ai = Al.numpy().astype(np.int64)
            bi = Bl.numpy().astype(np.int64)
            want = np.matmul(ai, np.swapaxes(bi, 1, 2))
            assert np.array_equal(Y, want.astype(np.float64)), (a, cd)
            assert np.array_equal(D, (want + Cl.numpy()).astype(np.float64))
            assert np.array_equal(S, np.matmul(np.abs(ai), np.swapaxes(np.abs(bi), 1, 2)))
    # uint8: every value 0..255, an int64 matmul; all-255 operands give
    # 255^2 K exactly (the largest products)
    Au = _rand("u8full", "u8", (L, M, K), 36)
    Bu = _rand("u8full", "u8", (L, N, K), 37)
    for b in "KN":
        D, Y, _ = run(orc, Au, store(Bu, "B", b), store(Cl, "C", "N"), M=M, N=N, K=K, L=L,
                      ab="u8", c="i32", b=b, alpha=2.0, beta=-1.0)
        want = np.matmul(Au.numpy().astype(np.int64), np.swapaxes(Bu.numpy().astype(np.int64), 1, 2))
        assert np.array_equal(Y, want.astype(np.float64)), b
        assert np.array_equal(D, (2 * want - Cl.numpy()).astype(np.float64)), b
    full = torch.full((L, M, K), 255, dtype=torch.uint8)
    fullb = torch.full((L, N, K), 255, dtype=torch.uint8)
    _, Y, _ = run(orc, full, fullb, M=M, N=N, K=K, L=L, ab="u8")
    assert np.all(Y == 255 * 255 * K)
    Af = _rand("int2", "f16", (L, M, K), 34)
    Bf = _rand("int2", "f16", (L, N, K), 35)
    _, Y, _ = run(orc, Af, Bf, M=M, N=N, K=K, L=L, ab="f16")
    want = np.matmul(Af.numpy().astype(np.int64), np.swapaxes(Bf.numpy().astype(np.int64), 1, 2))
    assert np.array_equal(Y, want.astype(np.float64))


def pin_library_fp64(orc):
    """An independent fp64 library matmul agrees to 1e-12 of S."""
    M, N, K, L = 33, 17, 257, 2
    for ab in FLOAT_AB:
        Al = _rand(_dist_for(ab), ab, (L, M, K), 41)
        Bl = _rand(_dist_for(ab), ab, (L, N, K), 42)
        _, Y, S = run(orc, Al, Bl, M=M, N=N, K=K, L=L, ab=ab)
        a64 = torch.from_numpy(lib_decode(Al).reshape(L, M, K))
        b64 = torch.from_numpy(lib_decode(Bl).reshape(L, N, K))
        want = torch.matmul(a64, b64.transpose(1, 2).contiguous()).numpy()
        assert np.all(np.abs(Y - want) <= 1e-12 * S), ab
        sw = torch.matmul(a64.abs(), b64.abs().transpose(1, 2).contiguous()).numpy()
        assert np.all(np.abs(S - sw) <= 1e-12 * sw), ab


def pin_majorness_duality(orc):
    """The same logical problem in every storage layout gives the same
    results, bit for bit (layout changes addressing, never arithmetic)."""
    M, N, K, L = 6, 10, 12, 2
    Al = _rand("normal", "f16", (L, M, K), 51)
    Bl = _rand("normal", "f16", (L, N, K), 52)
    Cl = _rand("normal", "f32", (L, M, N), 53)
    Xl = _rand("normal", "f16", (L, M, N), 54)
    ref = None
    for (a, b, cd) in LAYOUTS:
        out = run(orc, store(Al, "A", a), store(Bl, "B", b), store(Cl, "C", cd),
                  store(Xl, "X", cd), M=M, N=N, K=K, L=L, ab="f16", c="f32",
                  x="f16", a=a, b=b, cd=cd, alpha=2.0, beta=1.0, xf=3.0)
        if ref is None:
            ref = out
        for r, o in zip(ref, out):
            assert np.array_equal(r, o), (a, b, cd)


def pin_batch_independence(orc):
    """A batch of L equals L separate single-batch problems."""
    M, N, K, L = 5, 6, 20, 3
    Al = _rand("normal", "bf16", (L, M, K), 61)
    Bl = _rand("normal", "bf16", (L, N, K), 62)
    Cl = _rand("normal", "f32", (L, M, N), 63)
    D, Y, S = run(orc, Al, Bl, Cl, M=M, N=N, K=K, L=L, ab="bf16", c="f32",
                  alpha=1.0, beta=1.0)
    for l in range(L):
        d1, y1, s1 = run(orc, Al[l:l + 1].contiguous(), Bl[l:l + 1].contiguous(),
                         Cl[l:l + 1].contiguous(), M=M, N=N, K=K, L=1,
                         ab="bf16", c="f32", alpha=1.0, beta=1.0)
        assert np.array_equal(D[l], d1[0]) and np.array_equal(Y[l], y1[0]) \
            and np.array_equal(S[l], s1[0]), l


def pin_points_match_full(orc):
    """The listed-points entry point agrees with the full result."""
    M, N, K, L = 7, 9, 24, 2
    for cd in "NM":
        Al = _rand("e4m3tab", "e4m3", (L, K, M), 71)  # stored M-major
        Bl = _rand("e4m3tab", "e4m3", (L, K, N), 72)  # stored N-major
        Cl = _rand("normal", "f16", (L, M, N), 73)
        Cs = store(Cl, "C", cd)
        D, Y, S = orc.gemm_epi(M, N, K, L, Al, Bl, Cs, ab="e4m3", c="f16",
                               a_major="M", b_major="N", cd_major=cd,
                               alpha=0.25, beta=1.0, nthreads=3)
        pts = [(l, m, n) for l in range(L) for m in range(M) for n in range(N)
               if (l + 2 * m + 3 * n) % 4 == 0]
        d, y, s = orc.gemm_epi_points(M, N, K, L, Al, Bl, Cs, points=pts,
                                      ab="e4m3", c="f16", a_major="M",
                                      b_major="N", cd_major=cd, alpha=0.25,
                                      beta=1.0, nthreads=2)
        Dl = from_cd_layout(D, L, M, N, cd)
        Yl = from_cd_layout(Y, L, M, N, cd)
        Sl = from_cd_layout(S, L, M, N, cd)
        for i, (l, m, n) in enumerate(pts):
            assert d[i] == Dl[l, m, n] and y[i] == Yl[l, m, n] and s[i] == Sl[l, m, n]


def pin_linearity(orc):
    """D(alpha, beta, x) = alpha*Y + beta*C + x*X for exactly representable
    terms (small dyadic inputs keep every intermediate exact)."""
    M, N, K, L = 4, 5, 12, 1
    Al = _rand("small", "f16", (L, M, K), 81)
    Bl = _rand("small", "f16", (L, N, K), 82)
    Cl = _rand("small", "bf16", (L, M, N), 83)
    Xl = _rand("small", "f32", (L, M, N), 84)
    _, Y, _ = run(orc, Al, Bl, M=M, N=N, K=K, L=L, ab="f16")
    cv = lib_decode(Cl).reshape(L, M, N)
    xv = lib_decode(Xl).reshape(L, M, N)
    for (al, be, xf) in ((2.0, 1.0, 3.0), (-0.5, 4.0, 0.25), (1.0, -1.0, -1.0)):
        D, _, _ = run(orc, Al, Bl, Cl, Xl, M=M, N=N, K=K, L=L, ab="f16",
                      c="bf16", x="f32", alpha=al, beta=be, xf=xf)
        assert np.array_equal(D, al * Y + be * cv + xf * xv), (al, be, xf)


def pin_fp8_pairs(orc):
    """A and B in different fp8 formats (e4m3 x e5m2 and e5m2 x e4m3), every
    layout: exact rational arithmetic on each operand's own decoding."""
    M, N, K, L = 3, 4, 6, 1
    seed = 98000
    for at, bt in (("e4m3", "e5m2"), ("e5m2", "e4m3")):
        for (a, b, cd) in LAYOUTS:
            seed += 10
            Al = _rand(_dist_for(at), at, (L, M, K), seed + 1)
            Bl = _rand(_dist_for(bt), bt, (L, N, K), seed + 2)
            Cl = _rand("normal", "f16", (L, M, N), seed + 3)
            D, Y, _ = run(orc, store(Al, "A", a), store(Bl, "B", b), store(Cl, "C", cd), M=M,
                          N=N, K=K, L=L, ab=at, bt=bt, c="f16", a=a, b=b, cd=cd,
                          alpha=1.0, beta=0.5)
            av = lib_decode(Al).reshape(L, M, K)
            bv = lib_decode(Bl).reshape(L, N, K)
            cv = lib_decode(Cl).reshape(L, M, N)
            for m in range(M):
                for n in range(N):
                    acc = sum(Fraction(av[0, m, k]) * Fraction(bv[0, n, k]) for k in range(K))
                    assert Fraction(Y[0, m, n]) == acc, (at, bt, a, b, cd, m, n)
                    assert Fraction(D[0, m, n]) == acc + Fraction(0.5) * Fraction(cv[0, m, n]), \
                        (at, bt, a, b, cd, m, n)


# --------------------------------------------------------------------------
# the clamped epilogue: D = max(0, alpha*Y + beta*C) + x_factor*X (the form
# the example's epilogue function builds)
# --------------------------------------------------------------------------

def pin_relu_bruteforce(orc):
    """Tiny mixed-sign problems: the clamped form equals exact rational
    arithmetic (clamp at zero of alpha*Y + beta*C, then the X term), both
    majornesses of C/D/X, floating and integer inputs."""
    M, N, K, L = 4, 5, 6, 2
    seed = 95000
    for ab in ("f16", "i8"):
        for cd in "NM":
            seed += 10
            Al = _rand("int2" if ab == "f16" else "i8full", ab, (L, M, K), seed + 1)
            Bl = _rand("int2" if ab == "f16" else "i8full", ab, (L, N, K), seed + 2)
            c = x = "f32" if ab == "f16" else "i32"
            Cl = _rand("i1000" if ab == "i8" else "normal", c, (L, M, N), seed + 3)
            Xl = _rand("i1000" if ab == "i8" else "normal", x, (L, M, N), seed + 4)
            alpha, beta, xf = (1.5, -0.75, 2.0) if ab == "f16" else (3.0, -2.0, 5.0)
            D, _, _ = run(orc, Al, Bl, store(Cl, "C", cd), store(Xl, "X", cd), M=M, N=N,
                          K=K, L=L, ab=ab, c=c, x=x, cd=cd, alpha=alpha, beta=beta,
                          xf=xf, relu=True)
            av = lib_decode(Al).reshape(L, M, K)
            bv = lib_decode(Bl).reshape(L, N, K)
            cv = lib_decode(Cl).reshape(L, M, N)
            xv = lib_decode(Xl).reshape(L, M, N)
            clamped = 0
            for l in range(L):
                for m in range(M):
                    for n in range(N):
                        acc = sum(Fraction(av[l, m, k]) * Fraction(bv[l, n, k]) for k in range(K))
                        inner = Fraction(alpha) * acc + Fraction(beta) * Fraction(cv[l, m, n])
                        clamped += inner <= 0
                        want = max(inner, Fraction(0)) + Fraction(xf) * Fraction(xv[l, m, n])
                        assert abs(Fraction(D[l, m, n]) - want) <= abs(want) * Fraction(2.0 ** -50), \
                            (ab, cd, l, m, n)
            assert 0 < clamped < L * M * N, (ab, cd, clamped)  # both sides of the clamp occur


def pin_relu_sign_identity(orc):
    """max(0, v) + max(0, -v) = |v|: with the X term absent, the clamped form
    at (alpha, beta) plus the clamped form at (-alpha, -beta) equals the
    magnitude of the plain form, exactly (negation is exact)."""
    M, N, K, L = 6, 7, 40, 2
    Al = _rand("normal", "bf16", (L, M, K), 96001)
    Bl = _rand("normal", "bf16", (L, N, K), 96002)
    Cl = _rand("normal", "f32", (L, M, N), 96003)
    for cd in "NM":
        Cs = store(Cl, "C", cd)
        kw = dict(M=M, N=N, K=K, L=L, ab="bf16", c="f32", cd=cd)
        plain, _, _ = run(orc, Al, Bl, Cs, alpha=1.25, beta=-0.5, **kw)
        pos, _, _ = run(orc, Al, Bl, Cs, alpha=1.25, beta=-0.5, relu=True, **kw)
        neg, _, _ = run(orc, Al, Bl, Cs, alpha=-1.25, beta=0.5, relu=True, **kw)
        assert np.all(pos >= 0) and np.all(neg >= 0), cd
        assert np.array_equal(pos + neg, np.abs(plain)), cd
        assert np.array_equal(pos - neg, plain), cd


def pin_relu_closed_forms(orc):
    """Clamped form: a non-positive alpha*Y + beta*C leaves exactly
    x_factor*X; a non-negative one leaves exactly the plain form."""
    M, N, K, L = 5, 6, 24, 1
    Al = torch.from_numpy(np.abs(_rand("int2", "f16", (L, M, K), 97001).numpy()))
    Bl = torch.from_numpy(np.abs(_rand("int2", "f16", (L, N, K), 97002).numpy()))
    Cl = torch.from_numpy(np.abs(_rand("int2", "f16", (L, M, N), 97003).numpy()))
    Xl = _rand("normal", "f16", (L, M, N), 97004)
    kw = dict(M=M, N=N, K=K, L=L, ab="f16", c="f16", x="f16")
    xv = lib_decode(Xl).reshape(L, M, N)
    D, _, _ = run(orc, Al, Bl, Cl, Xl, alpha=-2.0, beta=-1.0, xf=3.0, relu=True, **kw)
    assert np.array_equal(D, 3.0 * xv)
    Dr, _, _ = run(orc, Al, Bl, Cl, Xl, alpha=2.0, beta=1.0, xf=3.0, relu=True, **kw)
    Dp, _, _ = run(orc, Al, Bl, Cl, Xl, alpha=2.0, beta=1.0, xf=3.0, **kw)
    assert np.array_equal(Dr, Dp)


ALL_PINS = [pin_decode_golden, pin_decode_vs_library, pin_bruteforce_exact,
            pin_identity_A, pin_identity_B, pin_all_ones, pin_rank1,
            pin_alpha_zero, pin_skip_and_identity_epilogue, pin_integer_exact,
            pin_library_fp64, pin_majorness_duality, pin_batch_independence,
            pin_points_match_full, pin_linearity, pin_fp8_pairs, pin_relu_bruteforce,
            pin_relu_sign_identity, pin_relu_closed_forms]

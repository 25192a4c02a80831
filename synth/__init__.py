"""Seeded synthetic inputs for the fused-epilogue GEMM workloads.

Shared by the tests, the bench and the oracle checks.  This module holds none
of the method's arithmetic: it only draws stored elements (with torch's CPU
generator) and knows the storage shape each majorness implies.  Values are
drawn in fp32 (or as integers) and rounded to the storage type by torch.

The five workloads are the example shapes of the CuTe DSL example
``custom_epilogue_dense_gemm.py`` (its "Example usage": 8192^3 fp16 with
alpha 2, beta 1, x_factor 3) plus the smaller, bf16, batched-int8 and fp8
cases the benchmark plan adds; their value distributions are fixed here.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch

TORCH_DTYPE = {
    "f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn,
    "e5m2": torch.float8_e5m2,
    "i8": torch.int8, "u8": torch.uint8, "f32": torch.float32, "i32": torch.int32,
}
ELEM_BYTES = {"f16": 2, "bf16": 2, "e4m3": 1, "e5m2": 1, "i8": 1, "u8": 1, "f32": 4, "i32": 4}


@dataclasses.dataclass(frozen=True)
class Problem:
    """One workload: shapes, layouts, storage types, scalars, distributions."""
    name: str
    M: int
    N: int
    K: int
    L: int
    ab: str
    a_major: str = "K"
    b_major: str = "K"
    cd_major: str = "N"
    c: Optional[str] = None
    x: Optional[str] = None
    d: str = "f32"
    y: Optional[str] = None
    alpha: float = 1.0
    beta: float = 0.0
    x_factor: float = 0.0
    dist_ab: str = "normal"
    dist_c: str = "normal"
    dist_x: str = "normal"
    seed: int = 0
    epilogue: str = "linear"  # or "relu": D = max(0, alpha*Y + beta*C) + x_factor*X
    b_ab: Optional[str] = None    # B's own type (fp8 pairs), else ab
    dist_b: Optional[str] = None  # B's distribution, else dist_ab

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.L

    def replace(self, **kw) -> "Problem":
        return dataclasses.replace(self, **kw)

    def storage_shape(self, which: str):
        """Shape of the packed storage of one operand (L outermost)."""
        M, N, K, L = self.M, self.N, self.K, self.L
        if which == "A":
            return (L, M, K) if self.a_major == "K" else (L, K, M)
        if which == "B":
            return (L, N, K) if self.b_major == "K" else (L, K, N)
        return (L, M, N) if self.cd_major == "N" else (L, N, M)

    def algorithmic_bytes(self) -> int:
        """Each input read once, each output written once (skipped terms
        are not counted)."""
        eb = ELEM_BYTES
        n = self.M * self.N * self.L
        total = eb[self.ab] * (self.M + self.N) * self.K * self.L
        if self.c and self.beta != 0.0:
            total += eb[self.c] * n
        if self.x and self.x_factor != 0.0:
            total += eb[self.x] * n
        total += eb[self.d] * n
        if self.y:
            total += eb[self.y] * n
        return total


# The five benchmark workloads (index 0..4) and one HBM-bound extra (5).
CONFIGS = [
    Problem("int_small_f16_128", 128, 128, 128, 1, "f16", c="f32", d="f32",
            alpha=1.5, beta=0.5, dist_ab="int2", dist_c="int2", seed=1000),
    Problem("bf16_4096_f32out", 4096, 4096, 4096, 1, "bf16", c="f32",
            d="f32", alpha=1.0, beta=1.0, dist_ab="normal", dist_c="normal",
            seed=2000),
    Problem("f16_8192_fused_cxdy", 8192, 8192, 8192, 1, "f16", c="f16",
            x="f16", d="f16", y="f16", alpha=2.0, beta=1.0, x_factor=3.0,
            dist_ab="unif", dist_c="unif", dist_x="unif", seed=3000),
    Problem("i8_4096x4_mmajorA", 4096, 4096, 4096, 4, "i8", a_major="M",
            c="i32", d="i32", alpha=1.0, beta=1.0, dist_ab="i8full",
            dist_c="i1000", seed=4000),
    Problem("e4m3_8192_f16out", 8192, 8192, 8192, 1, "e4m3", c="f16",
            d="f16", alpha=0.25, beta=1.0, dist_ab="e4m3tab", dist_c="normal",
            seed=5000),
    # Index 5, a reported extra: the fp16 fused workload at K = 256, where the
    # epilogue's C, X, D, Y traffic (512 MiB) dwarfs the 34 GFLOP of the
    # product, so the launch is HBM-bound.
    Problem("f16_8192x8192_k256_cxdy", 8192, 8192, 256, 1, "f16", c="f16",
            x="f16", d="f16", y="f16", alpha=2.0, beta=1.0, x_factor=3.0,
            dist_ab="unif", dist_c="unif", dist_x="unif", seed=7100),
]

_E4M3_TABLE = None


def e4m3_table() -> torch.Tensor:
    """All distinct finite e4m3fn values with |v| <= 4 (-0 folded into 0),
    found by decoding every one of the 256 codes with torch: 145 values."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
        vals = codes.view(torch.float8_e4m3fn).to(torch.float32)
        keep = torch.isfinite(vals) & (vals.abs() <= 4.0)
        uniq = torch.unique(vals[keep] + 0.0)  # +0.0 folds -0 into +0
        _E4M3_TABLE = uniq.to(torch.float8_e4m3fn)
    return _E4M3_TABLE


_E5M2_TABLE = None


def e5m2_table() -> torch.Tensor:
    """All distinct finite e5m2 values with |v| <= 4 (-0 folded into 0),
    found by decoding every one of the 256 codes with torch."""
    global _E5M2_TABLE
    if _E5M2_TABLE is None:
        codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
        vals = codes.view(torch.float8_e5m2).to(torch.float32)
        keep = torch.isfinite(vals) & (vals.abs() <= 4.0)
        uniq = torch.unique(vals[keep] + 0.0)
        _E5M2_TABLE = uniq.to(torch.float8_e5m2)
    return _E5M2_TABLE


def draw(dist: str, dtype: str, numel: int, seed: int) -> torch.Tensor:
    """``numel`` stored elements of ``dtype`` from distribution ``dist``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    td = TORCH_DTYPE[dtype]
    if dist == "int2":  # integers in [-2, 2]
        v = torch.randint(-2, 3, (numel,), generator=g, dtype=torch.int32)
        return v.to(td)
    if dist == "normal":
        v = torch.randn(numel, generator=g, dtype=torch.float32)
        return v.to(td)
    if dist == "unif":  # uniform [-1, 1)
        v = torch.rand(numel, generator=g, dtype=torch.float32) * 2.0 - 1.0
        return v.to(td)
    if dist == "i8full":  # integers in [-128, 127]
        v = torch.randint(-128, 128, (numel,), generator=g, dtype=torch.int32)
        return v.to(td)
    if dist == "u8full":  # integers in [0, 255]
        v = torch.randint(0, 256, (numel,), generator=g, dtype=torch.int32)
        return v.to(td)
    if dist == "i1000":  # integers in [-1000, 1000]
        v = torch.randint(-1000, 1001, (numel,), generator=g,
                          dtype=torch.int32)
        return v.to(td)
    if dist == "e4m3tab":  # uniform over the 145-entry table
        tab = e4m3_table()
        idx = torch.randint(0, tab.numel(), (numel,), generator=g)
        out = tab.view(torch.uint8)[idx].view(torch.float8_e4m3fn)
        return out if td == torch.float8_e4m3fn else out.to(td)
    if dist == "e5m2tab":  # uniform over the finite e5m2 values with |v| <= 4
        tab = e5m2_table()
        idx = torch.randint(0, tab.numel(), (numel,), generator=g)
        out = tab.view(torch.uint8)[idx].view(torch.float8_e5m2)
        return out if td == torch.float8_e5m2 else out.to(td)
    if dist == "small":  # integers in [-3, 3] scaled by 1/4: exact everywhere
        v = torch.randint(-3, 4, (numel,), generator=g, dtype=torch.int32)
        return (v.to(torch.float32) * 0.25).to(td)
    raise ValueError("unknown distribution %r" % dist)


def make_inputs(p: Problem) -> Dict[str, Optional[torch.Tensor]]:
    """Host tensors A, B, C, X in their packed storage shapes.  Seeds are
    p.seed + {A: 1, B: 2, C: 3, X: 4}."""
    out: Dict[str, Optional[torch.Tensor]] = {}
    for which, dt, dist, s in (("A", p.ab, p.dist_ab, 1),
                               ("B", p.b_ab or p.ab, p.dist_b or p.dist_ab, 2),
                               ("C", p.c, p.dist_c, 3),
                               ("X", p.x, p.dist_x, 4)):
        if dt is None:
            out[which] = None
            continue
        shape = p.storage_shape(which)
        n = shape[0] * shape[1] * shape[2]
        out[which] = draw(dist, dt, n, p.seed + s).view(shape)
    return out

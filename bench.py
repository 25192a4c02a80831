#!/usr/bin/env python3
"""Throughput of the fused-epilogue batched GEMM on one MI355X.

One step = one call of the whole hot path (persistent GEMM + fused epilogue,
a single kernel launch) on inputs already resident in HBM.  Default workload:
M = N = K = 8192, L = 1, fp16 A/B (K-major), fp16 C, X, D, Y (N-major),
alpha 2, beta 1, x_factor 3 -- the shape and scalars of the CuTe DSL
example's "Example usage".

Prints ONE JSON line with the metric, a roofline object for the kernel
(MFMA-bound: achieved TFLOP/s from HIP events around every launch, on the
stream the kernel runs on, against the datasheet dense peak) and the CPU
oracle timed on a bounded sample of the same workload as a baseline.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % of MFMA dense peak, 8192³ fp16 GEMM w/ fused epilogue"
# MI355X datasheet dense MFMA peaks, TFLOP/s (TOP/s for int8)
PEAK = {"f16": 2500.0, "bf16": 2500.0, "e4m3": 5000.0, "e5m2": 5000.0, "i8": 5000.0, "u8": 5000.0}
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for rel in ("beta_epilogue_amd/csrc/gemm_epi_kernel.hpp",
                "beta_epilogue_amd/csrc/gemm_epi.hip",
                "beta_epilogue_amd/csrc/gemm_epi_part.hip",
                "beta_epilogue_amd/csrc/gemm_epi_launch.hpp",
                "beta_epilogue_amd/csrc/gemm_epi_raster.hpp",
                "beta_epilogue_amd/csrc/gemm_epi_variants.inc"):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed counter runs, only while the
    kernel sources are the ones the counters were taken on."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(workload)
    if not e or e.get("kernel_source_sha") != kernel_source_sha():
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(p, ins, target_s: float):
    """The oracle, as it stands, on whole rows of D; scaled to TFLOP/s."""
    import numpy as np
    import oracle
    threads = oracle.host_threads()

    def rows_points(nrows):
        ms = np.linspace(0, p.M * p.L - 1, nrows).astype(np.int64)
        pts = np.empty((nrows * p.N, 3), np.int64)
        pts[:, 0] = np.repeat(ms // p.M, p.N)
        pts[:, 1] = np.repeat(ms % p.M, p.N)
        pts[:, 2] = np.tile(np.arange(p.N), nrows)
        return pts

    def timed(nrows):
        pts = rows_points(nrows)
        t0 = time.perf_counter()
        oracle.gemm_epi_points(p.M, p.N, p.K, p.L, ins["A"], ins["B"], ins["C"],
                               ins["X"], points=pts, ab=p.ab, c=p.c, x=p.x,
                               a_major=p.a_major, b_major=p.b_major,
                               cd_major=p.cd_major, alpha=p.alpha, beta=p.beta,
                               x_factor=p.x_factor, relu=p.epilogue == "relu",
                               nthreads=threads)
        return time.perf_counter() - t0

    r0 = max(1, threads)
    dt0 = timed(r0)
    rows = int(min(p.M * p.L, max(r0, r0 * target_s / max(dt0, 1e-3))))
    dt = timed(rows)
    flops = 2.0 * p.K * rows * p.N
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d whole rows of D (%d outputs, K=%d fp64 dot products "
                      "plus the epilogue each), %.1f s" % (rows, rows * p.N, p.K, dt)}


CEILING_TYPES = {"f16": 1, "bf16": 2, "e4m3": 3, "i8": 4}
CEILING_INSTR = {"f16": ("v_mfma_f32_32x32x16_f16", "v_mfma_f32_16x16x32_f16"),
                 "bf16": ("v_mfma_f32_32x32x16_bf16", "v_mfma_f32_16x16x32_bf16"),
                 "e4m3": ("v_mfma_scale_f32_32x32x64_f8f6f4", "v_mfma_scale_f32_16x16x128_f8f6f4"),
                 "i8": ("v_mfma_i32_32x32x32_i8", "v_mfma_i32_16x16x64_i8")}


def mfma_ceiling(iters: int = 80000, rounds: int = 3, kinds=("constant", "random"), blocks=(32, 16),
                 types=("f16",)):
    """Steady clock and rate of register-only MFMA streams (block 32: the
    32x32 instruction, block 16: the 16x16 one) with no memory traffic,
    constant vs random operands (libmfma_ceiling.so), alternated `rounds`
    times, for each operand type in `types` (f16, bf16, e4m3, i8)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "beta_epilogue_amd", "libmfma_ceiling.so"))
    fn = lib.mfma_ceiling_run_type
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double),
                   ctypes.POINTER(ctypes.c_double)]
    fn.restype = ctypes.c_int
    out = {}
    for t in types:
        # int8 and fp8 instructions do 2x and 4x the FLOP of the fp16 ones per
        # step; fewer steps keep every launch near the same length
        n = iters if t in ("f16", "bf16") else iters // 2
        runs = {"%s_%dx%d" % (k, b, b): [] for b in blocks for k in kinds}
        for _ in range(rounds):
            for blk in blocks:
                for kind, rnd in (("constant", 0), ("random", 1)):
                    key = "%s_%dx%d" % (kind, blk, blk)
                    if key not in runs:
                        continue
                    ms, ghz, tf = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
                    rc = fn(CEILING_TYPES[t], blk, rnd, n, 3, ctypes.byref(ms), ctypes.byref(ghz),
                            ctypes.byref(tf))
                    if rc != 0:
                        raise RuntimeError("mfma_ceiling_run_type failed with HIP error %d" % rc)
                    runs[key].append({"ms": round(ms.value, 3), "ghz": round(ghz.value, 3),
                                      "tflops": round(tf.value, 1)})
        res = {"instructions": {"32x32": CEILING_INSTR[t][0], "16x16": CEILING_INSTR[t][1]},
               "unit": "TOP/s" if t == "i8" else "TFLOP/s", "peak": PEAK[t]}
        for key, r in runs.items():
            res[key] = {"tflops": round(sum(x["tflops"] for x in r) / len(r), 1),
                        "ghz": round(sum(x["ghz"] for x in r) / len(r), 3), "runs": r}
        out[t] = res
    return {"metric": "register-only MFMA stream, 8 waves per CU, constant vs random operands", "types": out}


def attainable_rate(ab: str, achieved: float):
    """The faster random-operand stream of the workload's operand type, as
    measured now, and the kernel's fraction of it."""
    cr = mfma_ceiling(rounds=2, kinds=("random",), types=(ab,))["types"][ab]
    key, c = max(((k, v) for k, v in cr.items() if k.startswith("random_")), key=lambda kv: kv[1]["tflops"])
    return {"tflops": c["tflops"], "ghz": c["ghz"], "frac": round(achieved / c["tflops"], 4),
            "shape": key.split("_")[1], "instruction": cr["instructions"][key.split("_")[1]],
            "how": "the faster of the 32x32 and 16x16 register-only MFMA streams of this operand type on "
                   "every CU, seeded random operands, same run (bench.py --mfma-ceiling)"}


def attainable_copy_rate(nbytes: int, achieved_gbs: float, reps: int = 40):
    """HBM context for a bandwidth-bound workload: torch's device-to-device
    copy moving the same number of bytes (half read, half written), timed
    with HIP events over reps launches, and the kernel's fraction of it."""
    import torch
    n = max(nbytes // 2, 1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del a, b
    return {"gbs": round(gbs, 1), "frac": round(achieved_gbs / gbs, 4),
            "how": "torch device copy of the same bytes (read + written), %d launches, same run" % reps}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2,
                    help="workload index 0..4 (2 = 8192^3 fp16 with C, X, D, Y); 5 = the same at K=256 (HBM-bound)")
    ap.add_argument("--shape", default=None, metavar="M,N,K,L",
                    help="other sizes for the workload's types, layouts and scalars (a shape study, "
                         "not the metric's workload)")
    ap.add_argument("--a-major", choices=("K", "M"), default=None,
                    help="A's majorness instead of the workload's (a layout study)")
    ap.add_argument("--b-major", choices=("K", "N"), default=None,
                    help="B's majorness instead of the workload's (a layout study)")
    ap.add_argument("--cd-major", choices=("N", "M"), default=None,
                    help="C, X, D and Y majorness instead of the workload's (a layout study)")
    ap.add_argument("--e5m2", action="store_true",
                    help="with an e4m3 workload: e5m2 A and B (finite values with |v| <= 4)")
    ap.add_argument("--bf16-out", action="store_true",
                    help="bf16 D (and Y) instead of the workload's 16-bit float outputs")
    ap.add_argument("--inplace", action="store_true",
                    help="D written over C (same type and layout), as the library allows")
    ap.add_argument("--uint8", action="store_true",
                    help="with an int8 workload: the same shape and layouts with uint8 A and B "
                         "(integers in [0, 255])")
    ap.add_argument("--splits", type=int, default=0,
                    help="K slices per split tile (0: the library's choice; 1: no split)")
    ap.add_argument("--epilogue", choices=("linear", "relu"), default="linear",
                    help="relu: D = max(0, alpha*A.B^T + beta*C) + x_factor*X")
    ap.add_argument("--variant", default="-1",
                    help="kernel variant: table index or name (-1: the default for the workload)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure register-only MFMA streams (fp16, bf16, e4m3, int8) on every "
                         "CU with constant and with random operands (steady clock and rate)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the attainable-rate measurements (MFMA streams; a device copy of the same bytes for an HBM-bound workload)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes "
                         "--steps times (scales the HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print("bench.py runs on one GPU only (the GEMM is sharded "
                  "by output tiles with no exchange; see the design notes); "
                  "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import beta_epilogue_amd as ge

    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling(types=tuple(CEILING_TYPES))), flush=True)
        return

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration, dtype=torch.uint8, device="cuda")
        src.fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration, "steps": args.steps}))
        return

    p = synth.CONFIGS[args.config]
    if args.shape:
        M, N, Kd, L = (int(v) for v in args.shape.split(","))
        p = p.replace(name="%s_at_%dx%dx%dx%d" % (p.name, M, N, Kd, L), M=M, N=N, K=Kd, L=L)
    for attr, val in (("a_major", args.a_major), ("b_major", args.b_major), ("cd_major", args.cd_major)):
        if val and val != getattr(p, attr):
            p = p.replace(name="%s_%s%s" % (p.name, attr[0], val.lower()), **{attr: val})
    if args.e5m2:
        if p.ab != "e4m3":
            sys.exit("--e5m2 takes an e4m3 workload")
        p = p.replace(name=p.name.replace("e4m3", "e5m2", 1), ab="e5m2", dist_ab="e5m2tab")
    if args.bf16_out:
        if p.d not in ("f16", "bf16") or (p.y and p.y not in ("f16", "bf16")):
            sys.exit("--bf16-out takes a workload with 16-bit float outputs")
        p = p.replace(name=p.name + "_bf16out", d="bf16", y="bf16" if p.y else None)
    if args.inplace:
        if p.c != p.d:
            sys.exit("--inplace needs C and D of one type")
        p = p.replace(name=p.name + "_inplace")
    if args.uint8:
        if p.ab != "i8":
            sys.exit("--uint8 takes an int8 workload")
        p = p.replace(name=p.name.replace("i8", "u8", 1), ab="u8", dist_ab="u8full")
    if args.epilogue != "linear":
        p = p.replace(name=p.name + "_" + args.epilogue, epilogue=args.epilogue)
    print("bench: workload %s M=%d N=%d K=%d L=%d" % (p.name, p.M, p.N, p.K, p.L),
          file=sys.stderr, flush=True)
    ins = synth.make_inputs(p)
    dev = {k: (v.cuda() if v is not None else None) for k, v in ins.items()}
    shape = p.storage_shape("D")
    if args.inplace:
        D = dev["C"]  # every step updates C; its values grow but stay finite over a run
    else:
        D = torch.empty(shape, dtype=synth.TORCH_DTYPE[p.d], device="cuda")
    Y = torch.empty(shape, dtype=synth.TORCH_DTYPE[p.y], device="cuda") if p.y else None
    variant = args.variant
    if not variant.lstrip("-").isdigit():
        names = [ge.gemm_epi_variant_name(i) for i in range(ge.gemm_epi_variant_count())]
        variant = names.index(variant)
    g = ge.FusedGemm(p.M, p.N, p.K, p.L, ab=p.ab, a_major=p.a_major,
                     b_major=p.b_major, cd_major=p.cd_major, c=p.c, x=p.x,
                     d=p.d, y=p.y, variant=int(variant), epilogue=p.epilogue, splits=args.splits)
    plan = g.plan
    print("bench: plan %s, %d tiles, grid %d, %d K slice(s) on %d split tile(s), workspace %d bytes"
          % (plan["name"], plan["tiles"], plan["grid"], plan["splits"], plan["split_tiles"],
             plan["workspace_bytes"]), file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step():
        g(dev["A"], dev["B"], dev["C"], dev["X"], D=D, Y=Y, alpha=p.alpha,
          beta=p.beta, x_factor=p.x_factor, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    region_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = region_ms / K
    avg_launch_ms = sum(launch_ms) / K
    flops = p.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK[p.ab]
    print("bench: %d steps, %.4f ms/step (events), %.4f ms/launch avg, min %.4f "
          "max %.4f, wall %.3f s, %s" % (K, ms_per_step, avg_launch_ms,
                                         min(launch_ms), max(launch_ms), wall,
                                         plan["name"]), file=sys.stderr, flush=True)

    # The attainable MFMA rate on this machine for operands like the workload's
    # (random data; the power cap sets the clock), measured right after.
    abytes = p.algorithmic_bytes()
    mfma_bound = flops / abytes >= peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    attainable = None
    if p.ab in CEILING_TYPES and mfma_bound and not args.no_ceiling:
        attainable = attainable_rate(p.ab, achieved)

    # MFMA-bound unless the arithmetic intensity (FLOP per algorithmic byte)
    # is under the ridge point peak / HBM bandwidth; then GB/s against HBM.
    common = {"traffic": measured_traffic(p.name), "algorithmic_bytes": abytes,
              "kernel": plan["name"], "avg_launch_ms": round(avg_launch_ms, 5)}
    if mfma_bound:
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(achieved / peak, 4), **common,
                    "attainable_random_operands": attainable}
    else:
        gbs = abytes / (avg_launch_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), **common,
                    "tflops": round(achieved, 2),
                    "attainable_device_copy": None if args.no_ceiling else attainable_copy_rate(abytes, gbs)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(p, ins, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.ab,
        "data": "synthetic (seeded; distributions of the workload definition)",
        "config": {"workload": p.name, "M": p.M, "N": p.N, "K": p.K, "L": p.L,
                   "ab": p.ab, "a_major": p.a_major, "b_major": p.b_major,
                   "cd_major": p.cd_major, "c": p.c, "x": p.x, "d": p.d,
                   "y": p.y, "alpha": p.alpha, "beta": p.beta,
                   "x_factor": p.x_factor, "epilogue": p.epilogue,
                   "accumulate": "i32" if p.ab == "i8" else "f32"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "plan": plan,
    }
    print(json.dumps(out), flush=True)
    g.close()


if __name__ == "__main__":
    main()

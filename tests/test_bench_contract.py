"""bench.py's output contract: one JSON line with the metric, the roofline
object of the timed kernel and the CPU oracle baseline; one GPU only."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=240):
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                       capture_output=True, text=True, timeout=timeout)
    return r


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout.strip() == ""


@pytest.mark.parametrize("opts,msg", [
    (("--config", "2", "--uint8"), "--uint8 takes an int8 workload"),
    (("--config", "2", "--e5m2"), "--e5m2 takes an e4m3 workload"),
    (("--config", "3", "--bf16-out"), "--bf16-out takes a workload with 16-bit float outputs"),
], ids=["uint8", "e5m2", "bf16_out"])
def test_study_options_refuse_other_workloads(opts, msg):
    r = _bench(*opts, timeout=120)
    assert r.returncode != 0 and msg in r.stderr and r.stdout.strip() == ""


def _line(r):
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
def test_bench_line_small_workload_with_cpu_baseline():
    print("bench --config 0", file=sys.stderr, flush=True)
    d = _line(_bench("--config", "0", "--steps", "3", "--warmup", "1", "--cpu-seconds", "1",
                     "--no-ceiling"))
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"]
    r = d["roofline"]
    assert r["bound"] in ("mfma", "hbm") and r["unit"] in ("TFLOP/s", "GB/s")
    assert r["achieved"] > 0 and r["peak"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert "traffic" in r
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]


@pytest.mark.gpu
def test_bench_line_hbm_bound_shape():
    print("bench --config 5", file=sys.stderr, flush=True)
    d = _line(_bench("--config", "5", "--steps", "3", "--warmup", "1", "--no-cpu-baseline"))
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000
    cp = r["attainable_device_copy"]
    assert cp["gbs"] > 0 and abs(cp["frac"] - r["achieved"] / cp["gbs"]) < 1e-3
    assert d["cpu_baseline"] is None


@pytest.mark.gpu
def test_bench_study_options():
    print("bench --shape / --splits / --uint8", file=sys.stderr, flush=True)
    r = _bench("--config", "2", "--shape", "1024,1024,8192,1", "--steps", "2", "--warmup", "1",
               "--no-cpu-baseline", "--no-ceiling")
    d = _line(r)
    assert d["config"]["M"] == 1024 and d["config"]["K"] == 8192
    assert "128x128" in r.stderr and "4 K slice(s) on 64 split tile(s)" in r.stderr, r.stderr
    r = _bench("--config", "2", "--shape", "1024,1024,8192,1", "--splits", "1", "--steps", "2", "--warmup", "1",
               "--no-cpu-baseline", "--no-ceiling")
    _line(r)
    assert "1 K slice(s) on 0 split tile(s)" in r.stderr, r.stderr
    d = _line(_bench("--config", "3", "--uint8", "--shape", "512,512,512,1", "--steps", "2", "--warmup", "1",
                     "--cpu-seconds", "0.5", "--no-ceiling"))
    assert d["dtype"] == "u8" and d["config"]["workload"].startswith("u8_")
    assert d["cpu_baseline"]["value"] > 0
    r = _bench("--config", "2", "--a-major", "M", "--b-major", "N", "--shape", "520,264,392,2", "--steps", "2",
               "--warmup", "1", "--no-cpu-baseline", "--no-ceiling")
    d = _line(r)
    assert d["config"]["a_major"] == "M" and d["config"]["b_major"] == "N"
    assert "plan f16_mn_n_" in r.stderr, r.stderr


@pytest.mark.gpu
@pytest.mark.parametrize("opts,plan", [
    (("--config", "2", "--cd-major", "M"), "plan f16_kk_m_"),
    (("--config", "2", "--bf16-out"), "plan f16_kk_n_"),
    (("--config", "2", "--inplace", "--epilogue", "relu"), "plan f16_kk_n_"),
    (("--config", "4", "--e5m2"), "plan e5m2_kk_n_"),
], ids=["cd_m", "bf16_out", "inplace_relu", "e5m2"])
def test_bench_form_options(opts, plan):
    print("bench", *opts, file=sys.stderr, flush=True)
    r = _bench(*opts, "--shape", "520,264,400,2", "--steps", "2", "--warmup", "1", "--no-cpu-baseline",
               "--no-ceiling")
    d = _line(r)
    assert plan in r.stderr, r.stderr
    assert d["value"] > 0 and d["config"]["M"] == 520

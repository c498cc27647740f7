"""bench.py's output contract: one JSON line with the fields the benchmark
record needs, internally consistent (tokens/s against the step time, each
roofline fraction against its peak), the oracle's CPU rate in the same line,
and a refusal of more than one GPU.

The CPU tests run bench.py's argument check and its CPU-baseline helper; the
GPU tests run bench.py itself on the small workloads, as a child process."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields(oracle_lib):
    import bench
    import engram_synth as S

    w = S.WORKLOADS["tiny_fp32"]
    res = bench.cpu_baseline(w, S.Inputs(w), budget_s=0.2)
    assert set(res) == {"value", "unit", "cores", "kind", "sample"}
    assert res["value"] > 0 and res["unit"] == "tokens/s"
    assert res["cores"] == 1 and res["kind"] == "oracle"
    assert "tiny_fp32" in res["sample"]


def _run_bench(*args):
    r = subprocess.run([sys.executable, "-u", BENCH, *args], capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-3000:]
    return json.loads(lines[0])


def _check_roofline(rf):
    assert rf["bound"] in ("hbm", "mfma")
    assert rf["unit"] == ("GB/s" if rf["bound"] == "hbm" else "TFLOP/s")
    assert rf["achieved"] > 0 and rf["peak"] > 0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) <= 1e-3 + 1e-3 * rf["frac"]
    assert "traffic" in rf and (rf["traffic"] is None or rf["traffic"] > 0)


def _check_common(d, workload, steps, warmup, dtype):
    import bench

    assert d["metric"] == bench.METRIC
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["data"] == "synthetic" and d["dtype"] == dtype
    assert d["config"]["workload"] == workload
    n = d["config"]["tokens_per_step"]
    assert abs(d["value"] - n / (d["ms_per_step"] * 1e-3)) <= 0.01 * d["value"]
    _check_roofline(d["roofline"])
    sr = d["step_roofline"]
    assert 0 < sr["frac"] <= 1 and sr["bound"] in ("hbm", "mfma")
    for k in d["kernels"]:
        _check_roofline({**k, "traffic": None})


@pytest.mark.gpu
def test_forward_line():
    d = _run_bench("--config", "tiny_fp32", "--steps", "3", "--warmup", "1")
    _check_common(d, "tiny_fp32", 3, 1, "f32")
    # the dominant kernel is the one the roofline names
    dom = max(d["kernels"], key=lambda k: k["avg_us"])
    assert d["roofline"]["kernel"] == dom["name"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0


@pytest.mark.gpu
def test_decode_line():
    d = _run_bench("--config", "decode_b256", "--steps", "4", "--warmup", "1", "--no-cpu-baseline")
    _check_common(d, "decode_b256", 4, 1, "bf16")
    assert d["config"]["tokens_per_step"] == d["config"]["batch"] == 256
    assert [k["name"] for k in d["kernels"]] == ["hash_gather", "project_gate_gemm", "decode_tail"]
    assert "cpu_baseline" not in d

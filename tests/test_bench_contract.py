"""bench.py's command-line contract: one GPU only, no CPU fallback, and the
fields of its JSON line."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, timeout):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=timeout)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"], 120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_no_gpu_is_an_error_not_a_fallback():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run(["--steps", "1", "--warmup", "0", "--no-cpu-baseline"], 300)
    assert r.returncode != 0
    assert not [ln for ln in r.stdout.splitlines() if ln.startswith("{")]


@pytest.mark.gpu
def test_bench_line_fields():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    r = _run(["--steps", "20", "--warmup", "20", "--no-cpu-baseline"], 300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 20
    assert d["higher_is_better"] is True and d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["peak"] == 5000.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # value is 2MNK over the whole step, which also holds the two rotate+quant launches
    M, N, K = d["config"]["M"], d["config"]["N"], d["config"]["K"]
    assert abs(d["value"] - 2 * M * N * K / (d["ms_per_step"] * 1e-3) / 1e12) / d["value"] < 0.01
    assert d["value"] < rf["achieved"]
    # the online layer (activation rotate+quant + GEMM) sits between the two
    ol = d["online_layer"]
    assert d["value"] < ol["TOPS"] < rf["achieved"]
    assert abs(ol["ms"] - d["kernels"]["rotate_quant_act"]["avg_ms"] - d["kernels"]["w4a4_gemm"]["avg_ms"]) < 1e-4


def test_committed_gemm_profile_gives_the_traffic_figure():
    """The bench line's roofline.traffic comes from the committed q_proj GEMM
    profile while its source hash matches the current GEMM sources."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.profile_traffic("w4a4_gemm_qproj_had128", bench.src_hash("gemm.hip", "common.h", "tile.h"))
    assert t is not None and t > 0
    assert bench.profile_traffic("w4a4_gemm_qproj_had128", "0" * 16) is None

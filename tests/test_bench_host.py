"""Host-side checks of bench.py's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_times_the_oracle_on_a_sample():
    """The cpu_baseline leg runs the oracle on whole (batch, head, query tile)
    units of the workload and reports its useful-flop rate and thread count."""
    sys.path.insert(0, ROOT)
    import bench
    from partial_context_patch_amd import workloads as WL

    name = "pcpp_tiny_fp32"
    res = bench.cpu_baseline(name, WL.workload_inputs(name), budget_s=0.5)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s"
    assert res["value"] > 0 and res["cores"] >= 1
    assert "units of 8" in res["sample"]  # 2 heads x 4 strips


def test_tier0_baseline_times_the_brute_force_oracle():
    """The tier-0 entry of cpu_baseline runs the oracle's Python loops on a
    bounded sample of the tiny strip layer and reports a useful-flop rate."""
    sys.path.insert(0, ROOT)
    import bench

    res = bench.cpu_tier0(budget_s=0.3)
    assert res["kind"] == "oracle" and res["unit"] == "TFLOP/s" and res["value"] > 0
    assert "tier 0" in res["sample"] and "pcpp_tiny_fp32" in res["sample"]

"""Host-side parts of bench.py that need no GPU: the one-GPU guard and the
oracle baseline over a process pool."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr


def test_cpu_baseline_reports_the_oracle_over_a_process_pool():
    import bench
    import synth

    wl = synth.WORKLOADS[0]
    res = bench.cpu_baseline(wl, synth.make_inputs(wl), seconds_target=0.2)
    assert res["kind"] == "oracle" and res["unit"] == "ms"
    assert res["cores"] == min(bench.cpu_cores(), wl.width) >= 1
    assert res["value"] > 0
    assert f"W={wl.width}" in res["sample"] and f"{res['cores']} worker processes" in res["sample"]

"""bench.py's command-line contract that holds without a GPU: the benchmark
measures one GPU, so --gpus above 1 ends with an error line and a non-zero
status before any device work."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                        "--warmup", "0", "--cpu-budget", "0"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_cpu_identity_names_model_and_cores():
    sys.path.insert(0, ROOT)
    import bench
    s = bench.cpu_model()
    assert "logical CPUs available" in s

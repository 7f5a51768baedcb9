"""bench.py's command-line contract, on the CPU: the options the driver
passes are parsed as given (exact steps and warmup, the settling time), and
more than one GPU is refused with a message before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _args(argv):
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    try:
        sys.argv = ["bench.py"] + argv
        return bench.parse()
    finally:
        sys.argv = old


def test_driver_options_are_taken_as_given():
    a = _args(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert (a.gpus, a.steps, a.warmup) == (1, 20, 5)
    assert a.settle_ms == 300.0 and a.workload == "window" and not a.only
    a = _args(["--steps", "7", "--warmup", "0", "--settle-ms", "0", "--workload", "prefill"])
    assert (a.steps, a.warmup, a.settle_ms, a.workload) == (7, 0, 0.0, "prefill")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                        "--warmup", "0"], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or "{" not in r.stdout   # no result line

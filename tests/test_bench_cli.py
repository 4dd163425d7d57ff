"""bench.py's command line on the CPU: the one-GPU rule and the tuning-plan
option are checked before anything needs a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_unknown_plan_knob_is_refused():
    r = _bench("--plan", "no_such_knob=3")
    assert r.returncode == 2
    assert "expected KNOB=VALUE" in r.stderr
    r = _bench("--plan", "pass2_heads=four")
    assert r.returncode == 2

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


def test_profiles_were_taken_from_the_current_kernels():
    """Every committed profile summary names the hash of the kernel sources it
    was taken from; it must be the current one (the token-causal summaries
    hash the walk's source too), so that no figure in profiles/ describes
    kernels that have since changed."""
    sys.path.insert(0, ROOT)
    import bench
    current = {False: bench.kernel_source_hash(False), True: bench.kernel_source_hash(True)}
    pdir = os.path.join(ROOT, "profiles")
    checked = 0
    for name in sorted(os.listdir(pdir)):
        text = open(os.path.join(pdir, name)).read()
        for line in text.splitlines():
            if line.startswith("kernel_source_sha256:"):
                assert line.split(":", 1)[1].strip() == current["token_causal" in name], name
                checked += 1
    assert checked >= 30

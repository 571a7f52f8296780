"""Host checks of bench.py's command-line contract (no GPU): more than one GPU
is refused with a message and a non-zero status before any GPU work, and
the traffic figures are reported only for the kernel sources they were
measured on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode != 0 and "WORLD_SIZE=2" in r.stderr


def test_traffic_figures_follow_the_measured_sources():
    """A traffic figure is reported while its kernel source is the one the
    counters were taken on, and null after any change to it."""
    import bench
    for kernel, (src, sha, nbytes) in bench.MEASURED_TRAFFIC.items():
        if bench.source_hash(src) == sha:
            assert bench.measured_traffic(kernel) == nbytes
        else:
            assert bench.measured_traffic(kernel) is None

"""bench.py's command line on the CPU: it measures one GPU only and says so for any other
count, before it touches torch or a device."""
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


def test_traffic_figure_is_tied_to_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    digest = bench.kernel_sources_digest()
    assert len(digest) == 64 and digest == bench.kernel_sources_digest()
    t = bench.measured_traffic()
    assert t is None or t > 0

"""bench.py's contract on the host (no GPU): with more than one GPU asked for
it exits with a message saying it measures one GPU, before touching torch;
its help lists the workloads; the stored HBM-traffic figure is read only for
the decode kernel sources it was taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    for n in ("2", "8"):
        p = run("--gpus", n)
        assert p.returncode == 2, p.stderr
        assert "one GPU" in p.stderr
        assert p.stdout == ""


def test_help_lists_the_workloads():
    p = run("--help")
    assert p.returncode == 0
    for w in ("C3", "C4", "C5", "WRITE", "VERIFY", "BLOCKS", "PREFIX", "STREAM"):
        assert w in p.stdout


def test_stored_traffic_matches_the_current_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.stored_traffic(-1) is not None       # the committed summary is current
    assert bench.stored_traffic(512) is None          # taken in the balanced mode only

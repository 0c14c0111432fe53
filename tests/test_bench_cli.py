"""bench.py on the host: more than one GPU is refused before anything
touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_sclk_parse():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.sclk_mhz({"clocks": {"card0": {"pp_dpm_sclk": "1: 2007Mhz *"}}}) == 2007.0
    assert bench.sclk_mhz({"clocks": None}) is None
    assert bench.sclk_mhz(None) is None

"""Host-side pieces of bench.py: the shader-clock reader and the one-GPU guard."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def write(tmp_path, text):
    p = tmp_path / "pp_dpm_sclk"
    p.write_text(text)
    return str(p)


def test_sclk_marked_level(tmp_path):
    # the driver marks the level the clock sits at; under a power cap that is an intermediate value
    assert bench.read_sclk_mhz(write(tmp_path, "0: 500Mhz\n1: 1612Mhz *\n2: 2400Mhz\n")) == 1612.0


def test_sclk_deep_sleep_line(tmp_path):
    assert bench.read_sclk_mhz(write(tmp_path, "S: 96Mhz *\n0: 500Mhz\n1: 2400Mhz\n")) == 96.0


def test_sclk_unmarked_or_missing(tmp_path):
    assert bench.read_sclk_mhz(write(tmp_path, "0: 500Mhz\n1: 2400Mhz\n")) is None
    assert bench.read_sclk_mhz(write(tmp_path, "garbage *\n")) is None
    assert bench.read_sclk_mhz(str(tmp_path / "absent")) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)

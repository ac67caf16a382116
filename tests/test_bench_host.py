"""Host-side pieces of bench.py: the shader-clock reader, the one-GPU guard and
the HBM-traffic arithmetic from counter CSVs."""
import json
import os
import subprocess
import sys

import pytest

import bench
import dense_gemm_07_amd as dg

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


# ---- HBM traffic from rocprofv3 counter CSVs --------------------------------------

def counters(tmp_path, name, rows):
    """A counter-collection CSV in rocprofv3's column names: (kernel, counter, value) rows."""
    p = tmp_path / name
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
    lines += [f'"{i}","{k}","{c}","{v}"' for i, (k, c, v) in enumerate(rows)]
    p.write_text("\n".join(lines) + "\n")
    return str(p)


GEMM = "void dg::gemm_mfma_lds<dg::BF16, 256, 256, 64, 2, 4, 0, 1, 2, 0>(dg::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


def recorded(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    fetch = counters(tmp_path, "f.csv", [(GEMM, "FETCH_SIZE", v) for v in (102.0, 98.0, 100.0)]
                     + [("void other_kernel(float*)", "FETCH_SIZE", 9999.0)])
    write = counters(tmp_path, "w.csv", [(GEMM, "WRITE_SIZE", v) for v in (50.0, 50.0, 51.0)])
    # the calibration copy is the kernel dispatched most often; its FETCH_SIZE reads half the bytes
    cfetch = counters(tmp_path, "cf.csv", [(COPY, "FETCH_SIZE", 131072.0)] * 5 + [("void fill(int*)", "FETCH_SIZE", 1.0)])
    cwrite = counters(tmp_path, "cw.csv", [(COPY, "WRITE_SIZE", 262144.0)] * 5)
    bench.record_traffic("toy", fetch, write, cfetch, cwrite, 256, "cmd")
    return json.loads((tmp_path / "traffic_toy.json").read_text())


def test_record_traffic_scales_each_counter_by_the_copy(tmp_path, monkeypatch):
    rec = recorded(tmp_path, monkeypatch)
    assert rec["kernels"] == [GEMM]  # the other kernel's samples are not counted
    assert rec["fetch_size_kib_raw"] == 100.0 and rec["write_size_kib_raw"] == 50.0  # medians
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0  # 256 MiB = 262144 KiB
    assert rec["hbm_read_bytes_per_launch"] == 100 * 2 * 1024
    assert rec["hbm_write_bytes_per_launch"] == 50 * 1024
    assert rec["hbm_bytes_per_launch"] == 100 * 2 * 1024 + 50 * 1024
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()


def tile(bm, bn, bk):
    c = dg.Config()
    c.block_m, c.block_n, c.block_k = bm, bn, bk
    return c


def test_traffic_is_reported_only_for_the_source_it_was_taken_on(tmp_path, monkeypatch):
    rec = recorded(tmp_path, monkeypatch)
    assert bench.measured_traffic("toy", tile(256, 256, 64)) == rec["hbm_bytes_per_launch"]
    assert bench.measured_traffic("no_such_workload", tile(256, 256, 64)) is None
    # ... and only for the tile shape it was taken on
    assert bench.measured_traffic("toy", tile(256, 256, 32)) is None
    assert bench.measured_traffic("toy", tile(128, 256, 64)) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.measured_traffic("toy", tile(256, 256, 64)) is None


def test_counter_without_samples_is_an_error(tmp_path):
    empty = counters(tmp_path, "e.csv", [(COPY, "WRITE_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench._counter_median(empty, "FETCH_SIZE", "dg::gemm")


def test_sized_workload_names():
    from dense_gemm_07_amd import inputs
    w = inputs.find("gemm_2048x1024x512_f16")
    assert (w.M, w.N, w.K, w.in_dtype, w.out_dtype, w.b_colmajor) == (2048, 1024, 512, "f16", "f16", False)
    assert inputs.find("square_4096_bf16").M == 4096  # the tables come first
    for bad in ("gemm_2048x1024_bf16", "gemm_1x2x3_int8", "gemm_axbxc_bf16"):
        with pytest.raises(KeyError):
            inputs.find(bad)

"""Host logic of bench.py that runs without a GPU: the one-GPU guard, the source hash that keys
the traffic and counter records, and the traffic record's calibration by the probe's 1 GiB copy."""
import csv
import json
import os
import shutil
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CSRC = os.path.join(ROOT, "nvfp4_block_scaled_mxfp8_amd", "csrc")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""                      # no JSON line


def _copy_sources(dst):
    for name in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(CSRC, name), dst)


def test_source_hash_ignores_comments_not_code(tmp_path):
    _copy_sources(tmp_path)
    h0 = bench.kernel_source_hash(str(tmp_path))
    assert h0 == bench.kernel_source_hash()
    g = tmp_path / "gemm.hip"
    text = g.read_text()
    g.write_text("// a new line comment\n/* and a\n   block comment */\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash(str(tmp_path)) == h0
    g.write_text(text + "\nstatic int one_more_declaration;\n")
    assert bench.kernel_source_hash(str(tmp_path)) != h0


def _counter_csv(d, counter, rows):
    """rocprofv3-style counter_collection.csv with (kernel, KiB) per dispatch, in dispatch order."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (kernel, v) in enumerate(rows):
            w.writerow([i + 1, i + 1, kernel, counter, v])


def test_traffic_record_is_scaled_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE reads 512 MiB for the probe's 1 GiB copy (factor 2), WRITE_SIZE 1 GiB (factor 1):
    the GEMM's last dispatch is scaled by those factors, and the record holds only while the
    sources hash the same."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    gemm = "void gmlp::gemm_mx_kernel<0, 0, 0>(gmlp::GemmArgs)"
    quant = "void gmlp::mxfp8_quant_kernel<true, true>(unsigned short const*, long)"
    fetch = [("__amd_rocclr_copyBuffer", 524288.0), ("__amd_rocclr_copyBuffer", 524300.0),
             ("__amd_rocclr_copyBuffer", 3.0), (gemm, 400000.0), (gemm, 401000.0), (quant, 131072.0)]
    write = [("__amd_rocclr_copyBuffer", 1048576.0), ("__amd_rocclr_copyBuffer", 1048576.0),
             ("__amd_rocclr_copyBuffer", 0.5), (gemm, 262144.0), (gemm, 262150.0), (quant, 140000.0)]
    _counter_csv(tmp_path / "fetch", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "write", "WRITE_SIZE", write)
    bench.write_traffic(types.SimpleNamespace(config="mid"), str(tmp_path / "fetch"), str(tmp_path / "write"))
    from workloads import CONFIGS
    cfg = CONFIGS["mid"]
    shape = bench.dominant_shape(cfg, bench.config_splits(cfg))
    rec = json.load(open(bench.traffic_file(shape)))
    fscale = 1048576.0 / 524300.0                      # the largest copy's reading
    assert rec["fetch_scale"] == pytest.approx(fscale)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes"] == round(401000.0 * 1024 * fscale)     # the last GEMM dispatch
    assert rec["write_bytes"] == round(262150.0 * 1024)
    assert rec["bytes_per_launch"] == round(401000.0 * 1024 * fscale + 262150.0 * 1024)
    assert rec["quantize"]["fetch_bytes"] == round(131072.0 * 1024 * fscale)
    assert rec["source_sha256"] == bench.kernel_source_hash()
    assert bench.measured_traffic(shape) == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda csrc=None: "0" * 64)
    assert bench.measured_traffic(shape) is None           # sources changed since: not reported


def test_gemm_algorithmic_bytes_of_the_large_workload():
    """E4M3 A [65536, 4096] and B [128, 7168, 4096], their u32 scale words per 128 contraction
    elements, the bf16 output [65536, 7168]."""
    shape = {"E": 128, "M": 65536, "N": 7168, "K": 4096}
    a, b = 65536 * 4096, 128 * 7168 * 4096
    words = 4 * 32 * (65536 + 128 * 7168)
    c = 2 * 65536 * 7168
    assert bench.gemm_algorithmic_bytes(shape) == a + b + words + c == 5091885056

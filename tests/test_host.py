"""Host-side logic on the CPU: the sweep's correctness gate, its resumable
record file and config filter, and the benchmark's source hash, traffic
lookup and refusal of more than one GPU."""
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench
from gemv_fp16_amd import sweep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def f16bits(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def test_sweep_ulp_is_the_spacing_to_the_next_larger_magnitude():
    vals = np.array([1.0, 1.5, 2.0, 1000.0, 30000.0, 6.1e-5, 3e-6, 0.0, -3.0, -0.0], dtype=np.float16)
    mags = np.abs(vals)
    ref = (np.nextafter(mags, np.float16(np.inf)).astype(np.float64) - mags.astype(np.float64))
    assert np.array_equal(sweep._ulp(vals.view(np.uint16)), ref)


def test_sweep_gate_tolerance():
    """One fp16 ulp of the reference plus 1e-3 passes, two ulps at 100 do not."""
    ref = f16bits([100.0, 100.0])
    up1 = f16bits([100.0625, 99.9375])
    up2 = f16bits([100.125, 100.0])
    assert sweep._close(up1, ref)
    assert not sweep._close(up2, ref)
    assert sweep._close(f16bits([1.0 + 2 ** -9]), f16bits([1.0]))    # 2 ulps at 1.0 are inside 1e-3 + 1 ulp
    assert not sweep._close(f16bits([1.0 + 3 * 2 ** -10]), f16bits([1.0]))


def test_sweep_records_resume_after_a_cut_record(tmp_path, capsys):
    p = str(tmp_path / "sweep.jsonl")
    assert sweep._done(p) == set()
    r1 = {"op": "gemm", "shape": [8, 8, 8], "config": {"block_m": 64}, "tflops": 1.0}
    r2 = {"op": "gemm", "shape": [8, 8, 8], "config": {"block_m": 128}, "tflops": 2.0}
    sweep._emit(p, r1)
    with open(p, "a") as f:
        f.write('{"op": "gemm", "shape": [8, 8')          # an interrupted run's last record
    sweep._emit(p, r2)
    key = lambda r: json.dumps([r["op"], r["shape"], r["config"]], sort_keys=True)
    assert sweep._done(p) == {key(r1), key(r2)}
    assert len(open(p).read().splitlines()) == 3
    out = capsys.readouterr().out.splitlines()
    assert [json.loads(l) for l in out] == [r1, r2]


def test_sweep_config_filter():
    assert sweep._parse_only("") == set()
    assert sweep._parse_only("256,256,64,2,256;128,128,64,2,256,2") == {
        (256, 256, 64, 2, 256, 0), (128, 128, 64, 2, 256, 2)}


def _copy_sources(dst):
    csrc = os.path.join(ROOT, "gemv_fp16_amd", "csrc")
    os.makedirs(os.path.join(dst, "gemv_fp16_amd", "csrc"))
    for name in {n for v in bench.KERNEL_SOURCES.values() for n in v}:
        shutil.copy(os.path.join(csrc, name), os.path.join(dst, "gemv_fp16_amd", "csrc", name))


def test_source_hash_follows_the_kernel_sources(tmp_path, monkeypatch):
    _copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    assert h == {k: bench.kernel_source_hash(k) for k in bench.KERNEL_SOURCES}
    with open(os.path.join(str(tmp_path), "gemv_fp16_amd", "csrc", "gemv_kernel.hpp"), "a") as f:
        f.write("\n")
    assert bench.kernel_source_hash("gemv_kernel") != h["gemv_kernel"]
    assert bench.kernel_source_hash("gemm_nt_kernel") == h["gemm_nt_kernel"]   # not one of its sources


def test_traffic_record_is_used_only_on_its_own_sources(tmp_path, monkeypatch):
    _copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("gemv_kernel", "8192^2") is None               # no file
    os.makedirs(os.path.join(str(tmp_path), "profiles"))
    path = os.path.join(str(tmp_path), "profiles", "traffic.json")
    rec = {"bytes_per_launch": 134500000, "source_hash": bench.kernel_source_hash("gemv_kernel")}
    json.dump({"gemv_kernel|8192^2": rec}, open(path, "w"))
    assert bench.measured_traffic("gemv_kernel", "8192^2") == 134500000
    assert bench.measured_traffic("gemv_kernel", "1024^2") is None                # no record
    json.dump({"gemv_kernel|8192^2": dict(rec, source_hash="0" * 16)}, open(path, "w"))
    assert bench.measured_traffic("gemv_kernel", "8192^2") is None               # stale
    open(path, "w").write("{not json")
    assert bench.measured_traffic("gemv_kernel", "8192^2") is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""

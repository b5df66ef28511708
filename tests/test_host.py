"""Host-side logic on the CPU: the sweep's correctness gate, its resumable
record file and config filter, the benchmark's source hash, traffic lookup
and refusal of more than one GPU, and the timeline tool's arithmetic."""
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


def test_clock_sampler_reads_the_marked_dpm_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1487Mhz *\n2: 2400Mhz\n")
    cs = bench.ClockSampler(period_s=0.001)
    cs.path = str(f)
    assert cs._read() == 1487
    import time
    t0 = time.perf_counter()
    cs.start()
    time.sleep(0.05)
    r = cs.stop(t0, time.perf_counter())
    assert r["median"] == 1487 and r["min"] == 1487 and r["samples"] >= 1
    f.write_text("0: 500Mhz\n1: 158Mhz\n")          # no marked level
    assert cs._read() is None
    cs.path = None                                    # several or no GPUs: not sampled
    assert cs.start().stop() is None


def test_stats_and_copy_rotation():
    t = np.array([3.0, 1.0, 2.0, 4.0, 10.0]) * 1e-6
    s = bench.stats(t, work=2e-6 * 1e12)
    assert s["median_us"] == 3.0 and s["min_us"] == 1.0 and s["reps"] == 5
    assert s["p90_us"] == round(float(np.percentile(t, 90)) * 1e6, 3)
    assert s["mean_us"] == 4.0
    assert s["rate_median"] == round(2e6 / 3e-6 / 1e12, 2)
    # rotations exceed three MALLs where the cap allows
    assert bench.copies_for(256 << 20) == 3
    assert bench.copies_for(2 << 20, cap=256) == 256
    assert bench.copies_for(1 << 30) == 1


def test_sweep_expected_files_load_and_check_their_shape(tmp_path):
    """The committed oracle expected values are read with their shape; a
    file for another shape, or none, stops the sweep instead of gating on
    the wrong values."""
    ij, u, i = sweep.load_expected(sweep.expected_path("gemm", [8192, 8192, 8192]), [8192, 8192, 8192])
    assert ij.shape[1] == 2 and ij.shape[0] == u.size == i.size >= 3000
    assert ij.min() >= 0 and ij[:, 0].max() == 8191 and ij[:, 1].max() == 8191
    n, gu, gi = sweep.load_expected(sweep.expected_path("gemv", [8192, 8192]), [8192, 8192])
    assert np.array_equal(n[:, 0], np.arange(8192))
    with pytest.raises(SystemExit):
        sweep.load_expected(sweep.expected_path("gemm", [8192, 8192, 8192]), [4096, 8192, 8192])
    with pytest.raises(SystemExit):
        sweep.load_expected(str(tmp_path / "none.txt"), [1, 1, 1])


def test_sweep_expected_values_are_the_oracles():
    """Spot-check the stored GEMM entries against the oracle recomputed here
    from the same seeded rows."""
    import inputs
    import oracle
    ij, u, i = sweep.load_expected(sweep.expected_path("gemm", [8192, 8192, 8192]), [8192, 8192, 8192])
    pick = np.arange(0, ij.shape[0], 97)
    rows = sorted(set(ij[pick, 0]) | set(ij[pick, 1]))
    pos = {r: t for t, r in enumerate(rows)}
    for kind, want in (("uniform", u), ("integer", i)):
        A = inputs.rows_f16(kind, (8192, 8192), rows, 0, inputs.STREAM_A)
        B = inputs.rows_f16(kind, (8192, 8192), rows, 0, inputs.STREAM_B)
        sub = np.array([[pos[a], pos[b]] for a, b in ij[pick]], dtype=np.int64)
        got, _ = oracle.gemm_nt_entries(A, B, sub)
        assert np.array_equal(got, want[pick])


def test_resource_remarks_parse():
    from gemv_fp16_amd import build
    text = """x.hpp:3:1: remark: Function Name: _Z3foov [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     TotalSGPRs: 36 [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     VGPRs: 20 [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     AGPRs: 4 [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     ScratchSize [bytes/lane]: 12 [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     Occupancy [waves/SIMD]: 8 [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     VGPRs Spill: 2 [-Rpass-analysis=kernel-resource-usage]
x.hpp:3:1: remark:     LDS Size [bytes/block]: 0 [-Rpass-analysis=kernel-resource-usage]
y.hpp:9:1: remark: Function Name: _Z3barv [-Rpass-analysis=kernel-resource-usage]
y.hpp:9:1: remark:     VGPRs: 7 [-Rpass-analysis=kernel-resource-usage]
"""
    r = build.parse_resource_remarks(text)
    assert r["_Z3foov"] == {"sgprs": 36, "vgprs": 20, "agprs": 4, "scratch_bytes": 12,
                            "occupancy_waves_per_simd": 8, "sgpr_spills": 0, "vgpr_spills": 2,
                            "static_lds_bytes": 0}
    assert r["_Z3barv"] == {"vgprs": 7}
    from gemv_fp16_amd import resources
    assert resources.spills(r["_Z3foov"]) and not resources.spills({"scratch_bytes": 0, "vgpr_spills": 0})
    assert not resources.spills(None)
    cfg = {"block_m": 256, "block_n": 256, "block_k": 64, "stages": 2, "threads": 256, "schedule": 2}
    assert resources.gemm_kernel_name(cfg) == (
        "void gf::gemm_nt_kernel<gf::GemmCfg<256, 256, 64, 2, 256, 2, 0, 0>, 0, true>(gf::GemmArgs)")
    # the epilogue's per-wave transpose (4 waves x 128 x (128 + 8) fp16) outgrows the 2-stage ring
    assert resources.gemm_lds_bytes(cfg) == max(2 * (256 + 256) * 64 * 2, 4 * 128 * 136 * 2) == 139264


def test_compare_config_parsing():
    """--compare reads each config as 'default' or the op's value list, and
    refuses a list of the wrong length instead of guessing."""
    d = {"block_m": 256, "block_n": 256, "block_k": 64, "stages": 2, "threads": 256, "raster": 0, "schedule": 2}
    assert sweep._cfg_from("gemm", "default", d) == d
    assert sweep._cfg_from("gemm", "256,128,64,3,256,2,1", d) == {
        "block_m": 256, "block_n": 128, "block_k": 64, "stages": 3, "threads": 256, "schedule": 2, "raster": 1}
    assert sweep._cfg_from("sparse", "128,256,3,1", {}) == {"block_m": 128, "block_n": 256, "stages": 3, "raster": 1}
    assert sweep._cfg_from("gemv", "1,4,4,512", {}) == {"rows_per_wave": 1, "unroll": 4, "waves": 4, "blocks": 512}
    with pytest.raises(SystemExit):
        sweep._cfg_from("sparse", "128,256,3", {})


def test_timeline_row_reads_the_stamps():
    """The timeline tool's row from synthetic stamps: two workgroups whose
    main loops run 10 us (real-time counter, 100 MHz) over 15000 shader
    cycles, i.e. 1.5 GHz, across 32 K tiles of a 256 x 128 x 64 tile."""
    import numpy as np
    from gemv_fp16_amd import timeline
    rec = np.array([
        # entry, first tile landed, loop end, stores done, XCC, cycles at entry, first tile, loop end
        [1000, 1200, 2200, 2300, 3, 50000, 52000, 67000],
        [1010, 1210, 2210, 2350, 5, 80000, 82000, 97000],
    ], dtype=np.int64)
    cfg = (256, 128, 64, 3, 256, 2)
    cells = [c.strip() for c in timeline.row("8", cfg, rec, 32 * 64).strip("|").split("|")]
    assert cells[0] == "8" and cells[1] == "256x128x64 S3 sched 2" and cells[2] == "2"
    assert cells[3] == "13.5"                    # span: last store 2350 - first entry 1000, in us
    assert cells[5] == "2.00"                    # prologue: entry to first tile, 200 ticks
    assert cells[6].startswith("10.0 ")          # main loop 1000 ticks = 10 us
    assert cells[8].startswith("1.50 ")          # 15000 cycles over 10 us
    assert cells[9] == "469"                     # 15000 cycles / 32 K tiles
    # 2 * 256 * 128 * 64 flops at 1024 per cycle and SIMD over 4 SIMDs = 1024 cycles per K tile
    assert cells[10] == "%.0f %%" % (100 * 1024 / (15000 / 32))
    assert cells[11] == "3:13.0 5:13.5"


def test_timeline_per_xcd_lines():
    """One line per XCC from the same stamps: clock and cycles per K tile."""
    import numpy as np
    from gemv_fp16_amd import timeline
    rec = np.array([
        [1000, 1200, 2200, 2300, 3, 50000, 52000, 67000],
        [1010, 1210, 2210, 2350, 5, 80000, 82000, 97000],
    ], dtype=np.int64)
    lines = timeline.per_xcd(rec, 32 * 64, 64).splitlines()
    assert lines[2] == "| 3 | 1 | 13.0 | 10.0 | 1.500 | 469 |"
    assert lines[3] == "| 5 | 1 | 13.5 | 10.0 | 1.500 | 469 |"

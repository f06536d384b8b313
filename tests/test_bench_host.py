"""Host-side logic of bench.py that needs no GPU: the refusal of more than one
GPU and the derivation of HBM bytes per launch from rocprofv3 counter databases."""

from __future__ import annotations

import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

GIB_KIB = 1 << 20


def _db(folder, counter: str, dispatches):
    os.makedirs(folder, exist_ok=True)
    with sqlite3.connect(os.path.join(folder, "run_results.db")) as db:
        db.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, value real)")
        db.executemany("insert into counters_collection values (?, ?, ?, ?)",
                       [(i, name, counter, v) for i, (name, v) in enumerate(dispatches, 1)])


def _run(tmp_path, monkeypatch, fetch, write, backward):
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    _db(fd, "FETCH_SIZE", fetch)
    _db(wd, "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.traffic_from(fd, wd, "ring-128k-P16", "bf16", backward) == 0
    return json.loads(out.read_text())


def test_forward_traffic_scaled_by_the_calibration(tmp_path, monkeypatch):
    # the fetch counter reads half the bytes of the 1 GiB copy: every fetch is scaled by 2
    fetch = [("FillFunctor<float>", 10.0), ("__amd_rocclr_copyBuffer", GIB_KIB / 2),
             ("fold_bf16_kernel<128, 8>", 1000.0), ("fold_bf16_kernel<128, 8>", 3000.0),
             ("__amd_rocclr_copyBufferRectAligned", 9 * GIB_KIB)]
    write = [("FillFunctor<float>", GIB_KIB), ("__amd_rocclr_copyBuffer", GIB_KIB),
             ("fold_bf16_kernel<128, 8>", 500.0), ("fold_bf16_kernel<128, 8>", 700.0),
             ("__amd_rocclr_copyBufferRectAligned", 9 * GIB_KIB)]
    rec = _run(tmp_path, monkeypatch, fetch, write, backward=False)["ring-128k-P16"]
    assert rec["launches"] == 2
    assert rec["read_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["read_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == pytest.approx(600.0 * 1024)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"])
    assert rec["source_sha256_16"] == bench._source_hash("bf16")


def test_write_scale_comes_from_the_fill_before_the_copy(tmp_path, monkeypatch):
    # a larger elementwise write (a 2 GiB random fill) and a later fill must not be taken
    # for the calibration: only the last fill before the calibration copy counts
    fetch = [("distribution_elementwise", 5.0), ("FillFunctor<float>", 1.0),
             ("__amd_rocclr_copyBuffer", GIB_KIB / 2), ("bwd_dq_kernel<128, 8>", 100.0),
             ("bwd_dkdv_kernel<128, 8>", 300.0), ("FillFunctor<float>", 1.0)]
    write = [("distribution_elementwise", 2 * GIB_KIB), ("FillFunctor<float>", GIB_KIB),
             ("__amd_rocclr_copyBuffer", GIB_KIB), ("bwd_dq_kernel<128, 8>", 40.0),
             ("bwd_dkdv_kernel<128, 8>", 60.0), ("FillFunctor<float>", 4 * GIB_KIB)]
    rec = _run(tmp_path, monkeypatch, fetch, write, backward=True)["ring-128k-P16/backward"]
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["launches"] == 1  # one dQ + dK/dV pair
    assert rec["read_bytes_per_launch"] == pytest.approx(400.0 * 1024 * 2)
    assert rec["write_bytes_per_launch"] == pytest.approx(100.0 * 1024)
    assert rec["source_sha256_16"] == bench._source_hash("bf16", backward=True)


def test_traffic_is_dropped_when_the_source_changes(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps({"ring-128k-P16": {"hbm_bytes_per_launch": 7.0, "source_sha256_16": "0" * 16}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench._traffic("ring-128k-P16", "bf16") is None
    out.write_text(json.dumps({"ring-128k-P16": {"hbm_bytes_per_launch": 7.0,
                                                 "source_sha256_16": bench._source_hash("bf16")}}))
    assert bench._traffic("ring-128k-P16", "bf16") == 7.0
    assert bench._traffic("ring-128k-P16", "bf16", backward=True) is None


def test_d256_traffic_is_tied_to_the_fold_kernel_source(tmp_path, monkeypatch):
    """Every bf16 head dim (d = 64, 128, 256) runs fold_bf16_kernel of
    fold_bf16.hip: a d = 256 traffic entry is gated on that file's hash and
    turns null once the file changes."""
    import hashlib

    src = os.path.join(bench.ROOT, "blockwise_online_softmax_fold_amd", "csrc", "fold_bf16.hip")
    with open(src, "rb") as f:
        want = hashlib.sha256(f.read()).hexdigest()[:16]
    assert bench._source_hash("bf16", False, 256) == want
    assert bench._source_hash("bf16", False, 256) == bench._source_hash("bf16", False, 128)
    assert bench._source_hash("bf16", False, 256) != bench._source_hash("f32", False, 256)
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    path.write_text(json.dumps({"w5": {"hbm_bytes_per_launch": 5.0, "source_sha256_16": want}}))
    assert bench._traffic("w5", "bf16", False, 256) == 5.0
    path.write_text(json.dumps({"w5": {"hbm_bytes_per_launch": 5.0, "source_sha256_16": "0" * 16}}))
    assert bench._traffic("w5", "bf16", False, 256) is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_overlap_condition_matches_the_pages_a100_figures():
    """vibeengines.com "At the extremes": at 312 TFLOP/s over a ~300 GB/s link a
    block of about 1,000 tokens (312e12 / 300e9 = 1040) hides the transfer; at
    12.5 GB/s it takes about 25,000 (24,960)."""
    assert bench.min_block_for_overlap(312e12, 300e9) == pytest.approx(1040.0)
    assert bench.min_block_for_overlap(312e12, 12.5e9) == pytest.approx(24960.0)
    # 32-bit elements move twice the bytes: twice the block
    assert bench.min_block_for_overlap(312e12, 300e9, elem_bytes=4) == pytest.approx(2080.0)


@pytest.mark.parametrize("c,d", [(1040, 128), (1040, 64), (8192, 128), (520, 256)])
def test_links_needed_is_one_exactly_at_the_threshold(c, d):
    """At F = 312 TFLOP/s and B = 300 GB/s a c-token step needs c_min / c links:
    one link exactly at c = 1040 whatever d is, half at twice the block."""
    F, Bw = 312e12, 300e9
    flops = 4.0 * d * c * c
    kv_bytes = 2.0 * c * d * 2
    n = bench.links_needed(flops, flops / F, kv_bytes, Bw)
    assert n == pytest.approx(bench.min_block_for_overlap(F, Bw) / c)
    if c == 1040:
        assert n == pytest.approx(1.0)


def test_parity_figures_apply_the_bars():
    import numpy as np

    ref = np.linspace(-1, 1, 64).reshape(4, 16)
    ok = bench.parity_figures(ref + 1e-3, ref, "bf16")
    assert ok["within_bar"] and ok["max_abs"] == pytest.approx(1e-3)
    bad = ref.copy()
    bad[0, 0] += 0.05
    assert not bench.parity_figures(bad, ref, "bf16")["within_bar"]
    assert bench.parity_figures(ref * (1 + 5e-6), ref, "f32")["within_bar"]
    assert not bench.parity_figures(ref * (1 + 5e-5), ref, "f32")["within_bar"]


def test_clock_sampler_reads_sysfs_clock_and_power(tmp_path, monkeypatch):
    """The sampler takes the starred pp_dpm_sclk level as the clock and
    hwmon power1_input / power1_cap (microwatts) as watts."""
    dev = tmp_path / "card0" / "device"
    hw = dev / "hwmon" / "hwmon0"
    hw.mkdir(parents=True)
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1900Mhz *\n2: 2400Mhz\n")
    (hw / "power1_input").write_text("1395000000\n")
    (hw / "power1_cap").write_text("1400000000\n")
    import glob as _glob

    real_glob = _glob.glob
    monkeypatch.setattr(_glob, "glob", lambda pat, *a, **k: [str(dev / "pp_dpm_sclk")] if pat.endswith("pp_dpm_sclk")
                        else real_glob(pat, *a, **k))
    c = bench.ClockSampler()
    assert c.cap_w == 1400.0
    c.samples.append(c._read())
    c.watts.append(bench._read_watts(c.power_path))
    rec = c.summary(950.0, 2500.0)
    assert rec["median_mhz"] == 1900.0
    assert rec["peak_at_clock"] == round(2500.0 * 1900.0 / 2400.0, 1)
    assert rec["power"]["median_w"] == 1395.0 and rec["power"]["cap_w"] == 1400.0

"""bench.py's command line on a host without a GPU: the contract's single-GPU
exit, the argument parser, and its pure helpers."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_contract_flags():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--workload", "--batch", "--graph", "--frame", "--host-input"):
        assert flag in r.stdout, flag


def test_algorithmic_bytes_count_the_covered_samples():
    from full_reference_video_amd import synth
    wl = synth.WORKLOADS[4]
    # 2160p at scale 8: windows cover 3836 x 2156 samples of both 2-byte planes
    assert bench.algorithmic_bytes(wl, 8) == 2 * 3836 * 2156 * 2
    assert bench.covered_extent(3840, 8) == 3836
    assert bench.covered_extent(481, 2) == 481  # the last window's low half still fits


@pytest.mark.parametrize("w,h,s", [(576, 324, 1), (853, 481, 2), (3840, 2160, 8)])
def test_map_flops_count_the_valid_region(w, h, s):
    dw, dh = -(-w // s), -(-h // s)
    assert bench.ssim_map_flops_per_frame(w, h, s) == (dw - 10) * (dh - 10) * 199


def test_ms_flops_count_five_levels():
    total, lw, lh = 0, 3840, 2160
    for _ in range(5):
        total += (lw - 10) * (lh - 10) * 243
        lw, lh = lw // 2, lh // 2
    assert bench.ms_flops_per_frame(3840, 2160) == total


def test_recorded_traffic_scales_per_frame_and_checks_the_sources(tmp_path, monkeypatch):
    rec = {"workload": "float_ssim_3840x2160_10bit", "frames_per_launch": 32.0,
           "kernel_sources_sha256": bench.kernel_sources_sha256(),
           "fetch_bytes_per_launch": 3200, "write_bytes_per_launch": 320}
    p = tmp_path / "rec.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(p))
    assert bench.recorded_traffic("float_ssim_3840x2160_10bit", 16.0) == 1760
    assert bench.recorded_traffic("float_ssim_1920x1080_8bit", 32.0) is None
    rec["kernel_sources_sha256"] = "0" * 64
    p.write_text(json.dumps(rec))
    assert bench.recorded_traffic("float_ssim_3840x2160_10bit", 32.0) is None


def test_cpu_model_names_the_host_cpu():
    m = bench.cpu_model()
    assert isinstance(m, str) and m


def test_default_streams_per_path():
    assert bench.default_streams("float_ssim", 8) == 1
    assert bench.default_streams("float_ssim", 2) == 1
    assert bench.default_streams("float_ssim", 1) == 2
    assert bench.default_streams("ms_ssim", 1) == 1


def test_cpu_baselines_time_the_oracle():
    from full_reference_video_amd import synth
    wl = synth.WORKLOADS[1]
    host = [synth.FrameSource(1).pair(0)]
    for res, cores in ((bench.cpu_baseline(host, wl, 0.3), 1), (bench.cpu_baseline_all_cores(host, wl, 0.3, 2), 2)):
        assert res["kind"] == "oracle" and res["unit"] == "frames/s"
        assert res["cores"] == cores and res["value"] > 0
        assert bench.cpu_model() in res["sample"]

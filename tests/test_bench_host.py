"""Host-side logic of bench.py (CPU only): the algorithmic byte counts the
roofline divides by, the counter summaries and their source-hash guard, and
the refusal of a multi-GPU run."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("M,V,dtype,op,red,want", [
    # the workloads' algorithmic bytes: logits read (and written back), int64
    # targets, fp32 losses
    (64, 1000, "f32", "fwd", "mean", 256_516),
    (64, 1000, "f32", "fwd", "none", 256_768),
    (32768, 4096, "f32", "fwd", "mean", 537_133_060),
    (16384, 131072, "bf16", "fwd", "mean", 4_295_098_372),
    (16384, 131072, "bf16", "fwd_bwd", "mean", 8_590_065_668),
    (8192, 50257, "f16", "fwd", "mean", 823_476_228),
    (8192, 50257, "f16", "fwd_bwd", "mean", 1_646_886_916),
    (1048576, 128, "f32", "fwd", "none", 549_453_824),
    (1048576, 128, "f32", "fwd", "mean", 545_259_524),
])
def test_algorithmic_bytes(M, V, dtype, op, red, want):
    assert bench.alg_bytes(M, V, dtype, op, red) == want


def test_algorithmic_bytes_other_ops():
    M, V = 10, 100
    # backward from a saved lse: logits, targets and lse in, gradient out
    assert bench.alg_bytes(M, V, "bf16", "bwd", "mean") == 2 * M * V * 2 + 8 * M + 4 * M
    assert bench.alg_bytes(M, V, "f32", "softmax", "none") == 2 * M * V * 4
    assert bench.alg_bytes(M, V, "f32", "fwd_lse", "none") == M * V * 4 + 8 * M + 4 * M + 4 * M
    with pytest.raises(ValueError):
        bench.alg_bytes(M, V, "f32", "nope", "mean")


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_by_the_copy_and_checks_the_source(tmp_path, monkeypatch):
    copy = "void (anonymous namespace)::copy_kernel<4>((anonymous namespace)::V4*)"
    ce = "void cek::rows_kernel<0, 64, 16, 0, true, 1, 4>(cek::Params)"
    # KiB per dispatch; the copy moves 1 GiB each way and FETCH_SIZE reads half of it
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(copy, 512 * 1024), (copy, 512 * 1024), (ce, 262144), (ce, 262146)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(copy, 1024 * 1024), (ce, 1), (ce, 3)])
    text = bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "classifier",
                               "fwd", "mean", "rows_kernel<0, 64, 16, 0, true", "cmd")
    d = dict(line.split(" = ", 1) for line in text.splitlines() if " = " in line
             and not line.startswith("#"))
    assert float(d["fetch_scale"]) == pytest.approx(2.0)
    assert float(d["write_scale"]) == pytest.approx(1.0)
    # medians: fetch 262145 KiB x 2, write 2 KiB x 1
    assert int(d["hbm_bytes_per_launch"]) == 262145 * 1024 * 2 + 2 * 1024
    assert d["kernel_source_sha"] == bench.kernel_source_hash()

    path = tmp_path / "traffic.txt"
    path.write_text(text)
    monkeypatch.setattr(bench, "traffic_path", lambda *a: str(path))
    assert bench.load_traffic("classifier", "fwd", "mean") == 262145 * 1024 * 2 + 2 * 1024
    # taken on other kernel sources: not reported
    path.write_text(text.replace(bench.kernel_source_hash(), "0" * 16))
    assert bench.load_traffic("classifier", "fwd", "mean") is None


def test_traffic_summary_refuses_a_kernel_with_no_counter_rows(tmp_path):
    copy = "void (anonymous namespace)::copy_kernel<4>((anonymous namespace)::V4*)"
    ce = "void cek::rows_kernel<0, 64, 16, 0, true, 1, 4>(cek::Params)"
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 512 * 1024), (ce, 262144)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1024 * 1024), (ce, 1)])
    with pytest.raises(ValueError, match="wg_kernel"):
        bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "lmhead",
                            "fwd_bwd", "mean", "wg_kernel<2, 16, 16", "cmd")
    # no calibration copy in the run: also refused, by name
    _counter_csv(tmp_path / "f2.csv", "FETCH_SIZE", [(ce, 262144)])
    with pytest.raises(ValueError, match="calibration copy"):
        bench.summarize_pmc(str(tmp_path / "f2.csv"), str(tmp_path / "w.csv"), "classifier",
                            "fwd", "mean", "rows_kernel<0, 64, 16, 0, true", "cmd")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

"""Host-side checks of bench.py: the one-GPU guard and the rocprofv3 summary
parsing (fake CSV output in the layout rocprofv3 writes)."""

import csv
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


SPLIT = "void (anonymous namespace)::gemv_ssq_split_kernel<5, 2, true, 8>(SplitArgs)"
KEYS = "void (anonymous namespace)::verify_keys_kernel(unsigned long long const*, int, int const*, int*, int*)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int, float*)"


def test_summarize_profiles(tmp_path, monkeypatch):
    kt, fe, wr, out = (str(tmp_path / n) for n in ("kt", "fetch", "write", "out"))
    _write_csv(os.path.join(kt, "box", "kt_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[SPLIT, 10, 336000, 33600, 90.0, 33000, 34000], [KEYS, 10, 10000, 1000, 2.7, 900, 1100]])
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    calib_kib = bench.CALIB_BYTES / 1024 / 2.0  # counter reads half the true bytes
    _write_csv(os.path.join(fe, "box", "f_counter_collection.csv"), hdr,
               [[SPLIT, "FETCH_SIZE", 1000.0], [SPLIT, "FETCH_SIZE", 1002.0], [KEYS, "FETCH_SIZE", 4.0],
                [NEG, "FETCH_SIZE", calib_kib]])
    _write_csv(os.path.join(wr, "box", "w_counter_collection.csv"), hdr,
               [[SPLIT, "WRITE_SIZE", 100.0], [KEYS, "WRITE_SIZE", 2.0], [NEG, "WRITE_SIZE", calib_kib]])
    bench.summarize_profiles(kt, fe, wr, out)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", os.path.join(out, os.path.basename(bench.TRAFFIC_FILE)))
    monkeypatch.setattr(bench, "KT_FILE", os.path.join(out, os.path.basename(bench.KT_FILE)))
    t = bench.read_traffic()
    assert t is not None
    # (1001 + 4) KiB and (100 + 2) KiB per call, times the calibration factor 2
    assert t["fetch_bytes"] == round(1005.0 * 1024 * 2) and t["write_bytes"] == round(102.0 * 1024 * 2)
    assert t["bytes"] == t["fetch_bytes"] + t["write_bytes"]
    assert bench.read_kernel_avgs() == {"gemv_ssq_split_kernel<5, 2, true, 8>": 33.6, "verify_keys_kernel": 1.0}
    # a summary taken from other sources is not used
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.read_traffic() is None and bench.read_kernel_avgs() is None


def test_summarize_requires_each_step_kernel(tmp_path):
    kt, fe, wr, out = (str(tmp_path / n) for n in ("kt", "fetch", "write", "out"))
    _write_csv(os.path.join(kt, "k_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[SPLIT, 1, 1, 1, 100, 1, 1]])
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    for d, c in ((fe, "FETCH_SIZE"), (wr, "WRITE_SIZE")):
        _write_csv(os.path.join(d, "c_counter_collection.csv"), hdr, [[SPLIT, c, 1.0], [NEG, c, 1.0]])
    with pytest.raises(SystemExit):
        bench.summarize_profiles(kt, fe, wr, out)


def test_step_algorithmic_bytes():
    rows, cols = bench.ROWS, bench.COLS
    assert bench.step_algo_bytes() == rows * cols // 32 * 68 + 8 * cols + 8 * rows + 20


def test_summarize_hit_rate(tmp_path, monkeypatch):
    d, out = str(tmp_path / "tcc"), str(tmp_path / "out")
    rows = []
    for i, k in enumerate(bench.HIT_KERNELS):
        for _ in range(2):
            rows += [[f"void (anonymous namespace)::{k}(Args)", "TCC_HIT_sum", 10.0 * (i + 1)],
                     [f"void (anonymous namespace)::{k}(Args)", "TCC_MISS_sum", 90.0]]
    _write_csv(os.path.join(d, "box", "tcc_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               rows)
    bench.summarize_hit_rate(d, out)
    monkeypatch.setattr(bench, "HIT_FILE", os.path.join(out, os.path.basename(bench.HIT_FILE)))
    r = bench.read_hit_rates()
    assert r is not None and set(r) == set(bench.HIT_KERNELS)
    for i, k in enumerate(bench.HIT_KERNELS):
        assert r[k] == round(10.0 * (i + 1) / (10.0 * (i + 1) + 90.0), 4)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.read_hit_rates() is None


def test_summarize_hit_rate_requires_each_kernel(tmp_path):
    d = str(tmp_path / "tcc")
    k = next(iter(bench.HIT_KERNELS))
    _write_csv(os.path.join(d, "c_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[k, "TCC_HIT_sum", 1.0], [k, "TCC_MISS_sum", 1.0]])
    with pytest.raises(SystemExit):
        bench.summarize_hit_rate(d, str(tmp_path / "out"))

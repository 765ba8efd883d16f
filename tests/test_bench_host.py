"""Host-side checks of bench.py: the one-GPU guard and the rocprofv3 summary
parsing (fake CSV output in the layout rocprofv3 writes), and the staleness
rule that drops a profile taken from other kernel sources."""

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


COMBINE = "void (anonymous namespace)::attn_combine_kernel<128>((anonymous namespace)::AttnArgs)"


def _isolated_dirs(tmp_path, name, kernel, dur_ns, fetch_kib, write_kib, hits, misses, valu):
    kt, fe, wr, sq = (str(tmp_path / name / n) for n in ("kt", "fetch", "write", "sq"))
    tr_hdr = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    second = {"step": KEYS}.get(name, COMBINE if name.startswith("attn") else None)
    rows, t = [], 1000
    for _ in range(bench.ISOLATED_CALLS):
        rows.append(["KERNEL_DISPATCH", kernel, t, t + dur_ns])
        if second:
            rows.append(["KERNEL_DISPATCH", second, t + dur_ns + 500, t + dur_ns + 2500])
        t += 100000
    _write_csv(os.path.join(kt, "box", "kt_kernel_trace.csv"), tr_hdr, rows)
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    calib_kib = bench.CALIB_BYTES / 1024 / 2.0  # the counter reads half the true bytes
    extra = [[COMBINE, "FETCH_SIZE", 10.0], [COMBINE, "WRITE_SIZE", 4.0]] if name.startswith("attn") else []
    _write_csv(os.path.join(fe, "box", "f_counter_collection.csv"), hdr,
               [[kernel, "FETCH_SIZE", fetch_kib], [kernel, "FETCH_SIZE", fetch_kib + 2], [NEG, "FETCH_SIZE", calib_kib]]
               + extra[:1])
    _write_csv(os.path.join(wr, "box", "w_counter_collection.csv"), hdr,
               [[kernel, "WRITE_SIZE", write_kib], [NEG, "WRITE_SIZE", calib_kib],
                [kernel, "TCC_HIT_sum", hits], [kernel, "TCC_MISS_sum", misses]] + extra[1:])
    _write_csv(os.path.join(sq, "box", "s_counter_collection.csv"), hdr,
               [[kernel, c, valu if c == "SQ_INSTS_VALU" else 1000.0]
                for c in bench.SQ_COUNTERS + ("GRBM_GUI_ACTIVE",)])
    return kt, fe, wr, sq


@pytest.mark.parametrize("name", ["q8n1", "step"])
def test_summarize_isolated(tmp_path, monkeypatch, name):
    kernel = "void (anonymous namespace)::" + bench.ISOLATED[name][1] + "(SplitArgs)"
    kt, fe, wr, sq = _isolated_dirs(tmp_path, name, kernel, 20000, 1000.0, 100.0, 25.0, 75.0, 3.2e6)
    out = str(tmp_path / "out")
    bench.summarize_isolated(name, kt, fe, wr, wr, sq, out)
    monkeypatch.setattr(bench, "isolated_profile_path", lambda n: os.path.join(out, f"gemv_{n}_17408x5120_isolated.txt"))
    kv = bench.read_isolated(name)
    assert kv is not None
    assert float(kv["duration_us_median"]) == 20.0
    # (1000 + 1002) / 2 KiB fetched, 100 KiB written, each times the calibration factor 2
    assert int(kv["fetch_bytes_per_launch"]) == round(1001.0 * 1024 * 2)
    assert int(kv["write_bytes_per_launch"]) == round(100.0 * 1024 * 2)
    assert float(kv["l2_hit_rate"]) == 0.25
    weights = bench.ROWS * bench.COLS * (2 if name == "step" else 1)
    assert abs(float(kv["valu_lane_ops_per_weight"]) - 3.2e6 * 64 / weights) < 1e-3
    if name == "step":  # GEMV start to verify end: 20 + 0.5 + 2 us
        assert float(kv["call_span_us_median"].split()[0]) == 22.5
    r = bench.isolated_roofline(name, bench.isolated_algo_bytes(name), 25.0)
    assert r["traffic"] == int(kv["traffic_bytes_per_launch"]) and r["rocprof_median_us"] == 20.0
    # a profile taken from other kernel sources is not used
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a: "0" * 64)
    assert bench.read_isolated(name) is None and bench.isolated_roofline(name, 1, 1.0)["traffic"] is None


def test_summarize_isolated_attention(tmp_path, monkeypatch):
    """Attention: pass 1's time, pass 2's time and the call span, traffic of
    both passes, no per-weight line, keyed to the attention source."""
    name = "attn4k"
    kernel = "void (anonymous namespace)::" + bench.ISOLATED[name][1] + "((anonymous namespace)::AttnArgs)"
    kt, fe, wr, sq = _isolated_dirs(tmp_path, name, kernel, 10000, 1000.0, 100.0, 25.0, 75.0, 3.2e6)
    out = str(tmp_path / "out")
    bench.summarize_isolated(name, kt, fe, wr, wr, sq, out)
    orig = bench.isolated_profile_path
    monkeypatch.setattr(bench, "isolated_profile_path", lambda n: os.path.join(out, os.path.basename(orig(n))))
    kv = bench.read_isolated(name)
    assert kv is not None and float(kv["duration_us_median"]) == 10.0
    assert float(kv["call_span_us_median"].split()[0]) == 12.5  # pass 1 start to pass 2 end
    assert int(kv["fetch_bytes_per_launch"]) == round((1001.0 + 10.0) * 1024 * 2)
    assert int(kv["write_bytes_per_launch"]) == round((100.0 + 4.0) * 1024 * 2)
    assert "valu_lane_ops_per_weight" not in kv and "valu_busy_frac" in kv
    assert kv["kernel_source_sha256"] == bench.kernel_source_hash(bench.ATTN_SOURCES)
    assert bench.isolated_algo_bytes(name) == bench.attn_algo_bytes(4096) == 33648640
    r = bench.isolated_roofline(name, bench.attn_algo_bytes(4096), 13.0)
    assert r["rocprof_call_span_us"] == 12.5 and r["traffic"] == int(kv["traffic_bytes_per_launch"])


def test_summarize_isolated_requires_every_dispatch(tmp_path):
    kernel = "void (anonymous namespace)::" + bench.ISOLATED["q8n4"][1] + "(GemvArgs)"
    kt, fe, wr, sq = _isolated_dirs(tmp_path, "q8n4", kernel, 20000, 1.0, 1.0, 1.0, 1.0, 1.0)
    other = "void (anonymous namespace)::" + bench.ISOLATED["q8n1"][1] + "(SplitArgs)"
    with pytest.raises(SystemExit):
        bench.summarize_isolated("q8n1", kt, fe, wr, wr, sq, str(tmp_path / "out"))  # kernel name mismatch
    assert other != kernel


def test_summarize_kt(tmp_path, monkeypatch):
    kt, out = str(tmp_path / "kt"), str(tmp_path / "out")
    _write_csv(os.path.join(kt, "box", "kt_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[SPLIT, 10, 336000, 33600, 90.0, 33000, 34000], [KEYS, 10, 10000, 1000, 2.7, 900, 1100]])
    bench.summarize_kt(kt, out)
    monkeypatch.setattr(bench, "KT_FILE", os.path.join(out, os.path.basename(bench.KT_FILE)))
    assert bench.read_kt_avg(bench.STEP_KERNEL) == 33.6
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a: "0" * 64)
    assert bench.read_kt_avg(bench.STEP_KERNEL) is None


def test_step_algorithmic_bytes():
    rows, cols = bench.ROWS, bench.COLS
    assert bench.step_algo_bytes() == rows * cols // 32 * 68 + 8 * cols + 8 * rows + 20
    assert bench.isolated_algo_bytes("step") == bench.step_algo_bytes()
    assert bench.isolated_algo_bytes("q8n4") == rows * cols // 32 * 34 + 4 * (rows + cols) * 4


def test_isolated_commands_run_committed_files():
    for name in bench.ISOLATED:
        cmds = bench.isolated_cmds(name)
        assert all("bench.py" in c for c in cmds.values())
        assert f"--only {name}" in cmds["kt"] and "--copy-calibration" in cmds["fetch"]

"""Benchmark of the packed-twin decode path on one MI355X.

A step is one pass of the hot path over one batch of synthetic input: the SSQ
twin GEMV over a 17408 x 5120 packed twin matrix (both twins' outputs from one
pass over the weights) with the greedy verify of the two output vectors fused
in (pti_gemv_ssq_verify: the GEMV kernel keeps each workgroup's largest
output, and a one-workgroup kernel reduces those).  ``value`` is effective weight bandwidth: packed weight bytes per
step / step time, with inputs resident in HBM.  The weights rotate over three
copies (568 MB, more than twice the 256 MB Infinity Cache), so every step
reads its weights from HBM.

Also reported on the same JSON line:
  * roofline: the step's entry point, both its kernels with the gap between
    them (algorithmic bytes per call / its time, the median over 10 runs of
    200 back-to-back calls timed with HIP events on its stream) against 8 TB/s
    HBM, its HBM traffic (both kernels) from the committed PMC summary, the
    kernels' own rocprofv3 averages from the committed kernel-trace summary,
    their L2 hit rates from the committed TCC summary, and its rate against
    a device-to-device copy of the same bytes (copy_ceiling);
  * per_kernel: the unfused pair (pti_gemv_ssq, then pti_verify_argmax), and
    the Q8 multi-stream GEMV over 17408 x 5120 at N = 1, 2, 4 streams
    (effective weight GB/s, GEMV/s, L2 hit rate, and t(N=4)/t(N=1)), each
    with median / p10 / p90 over 10 runs; a decoder layer's seven GEMVs separate, grouped
    and grouped in a graph; the toy decoder's forward pass eager and as a
    graph; twin-KV attention; the greedy and sampled verify at the toy
    decoder's vocabulary; the host packer;
  * cpu_baseline: the fp64 oracle (scalar C, one host core) running the same
    SSQ GEMV, timed on a bounded number of passes, with the host's CPU model
    and the same oracle code split over host threads beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROWS, COLS = 17408, 5120
HBM_PEAK_GBS = 8000.0
METRIC = "effective weight GB/s (% of 8 TB/s) + GEMV/s, 17408x5120 SSQ/Q8, N=1,2,4 streams"
MALL_BYTES = 256 * 2**20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# GPU outputs of each configuration, kept on the host for the CPU-baseline leg,
# which computes the oracle's results on the same inputs, times them, and
# reports the largest |y_gpu - y_oracle| / T (T = sum |scale q x| per output).
GPU_OUT = {}


def copies_for(nbytes: int) -> int:
    """Copies of a buffer to rotate through so the set is >= 2x the Infinity Cache."""
    return max(2, -(-2 * MALL_BYTES // nbytes))


def timed_loop(torch, fn, n_iter, stream, i0=0):
    """Average ms per call of fn(i) for i in range(i0, i0 + n_iter), HIP events on `stream`."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(i0, i0 + n_iter):
        fn(i)
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / n_iter


def timed_stats(torch, fn, stream, reps=10, per_rep=200, warmup=50):
    """Per-call time over `reps` back-to-back runs of `per_rep` calls each (after
    `warmup` calls): median, p10 and p90 in microseconds."""
    for i in range(warmup):
        fn(i)
    t = sorted(timed_loop(torch, fn, per_rep, stream, i0=r * per_rep) * 1e3 for r in range(reps))
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return {"median_us": round(q(0.5), 3), "p10_us": round(q(0.1), 3), "p90_us": round(q(0.9), 3)}


def graph_us(torch, pti, make, calls=50, reps=10):
    """GPU time per call with the host's launch cost taken out: `calls` calls,
    made by make(stream_handle)(i), captured on a side stream into one graph
    and replayed back to back; the median over `reps` replays, in
    microseconds.  (A call of a few microseconds timed in a Python loop is
    bound by the loop, not by the GPU.)"""
    s = torch.cuda.Stream()
    fn = make(pti._stream(s))
    torch.cuda.synchronize()
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    t = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(cur)
        g.replay()
        b.record(cur)
        b.synchronize()
        t.append(a.elapsed_time(b) * 1e3 / calls)
    del g
    t.sort()
    return round(t[len(t) // 2], 3)


def cpu_baseline(d, budget_s: float):
    """The oracle (scalar fp64 C, one thread) on the same SSQ GEMV, repeated
    until budget_s seconds have passed (at least once)."""
    import oracle
    P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.gemv_ssq(P, ROWS, COLS, d["xA"], d["xB"])
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per = el / n
    out = {"value": round(P.nbytes / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{n} full {ROWS}x{COLS} SSQ twin GEMVs (both twins), scalar fp64 C oracle, "
                     f"{per:.3f} s each, {el:.1f} s total",
           "gemv_per_s": round(1.0 / per, 4), "host_nproc": os.cpu_count(), "host_cpu": _cpu_model()}
    # the same per-row oracle code with the rows split over host threads (the
    # C call releases the GIL), for about half the budget
    from concurrent.futures import ThreadPoolExecutor
    nt = max(1, min(os.cpu_count() or 1, 16))
    parts = np.array_split(np.arange(ROWS, dtype=np.int64), nt)
    t0 = time.perf_counter()
    n = 0
    with ThreadPoolExecutor(nt) as ex:
        while True:
            list(ex.map(lambda idx: oracle.gemv_ssq_rows(P, ROWS, COLS, d["xA"], d["xB"], idx), parts))
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s / 2:
                break
    per = el / n
    out["threaded"] = {"value": round(P.nbytes / per / 1e9, 4), "unit": "GB/s", "cores": nt,
                       "sample": f"{n} full GEMVs, rows split over {nt} threads, {per:.3f} s each",
                       "gemv_per_s": round(1.0 / per, 4)}
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


HERE = os.path.dirname(os.path.abspath(__file__))
KT_FILE = os.path.join(HERE, "profiles", "bench_default_17408x5120_kernel_stats.md")
# the kernel of the headline step (the fused SSQ twin GEMV; verify_keys_kernel follows it)
STEP_KERNEL = "gemv_ssq_split_kernel<5, 2, true, 8>"
KERNEL_SOURCES = ("packed_twin_int8_amd/csrc/pti_gemv.hip", "packed_twin_int8_amd/csrc/pti_norm.h",
                  "packed_twin_int8_amd/csrc/pti_silu.h", "packed_twin_int8_amd/build.py")
ATTN_SOURCES = ("packed_twin_int8_amd/csrc/pti_attn.hip", "packed_twin_int8_amd/build.py")
KT_CMDS = {
    "kt": "rocprofv3 --kernel-trace --stats -f csv -d rocprof_out/bench -o bench -- python3 bench.py --no-cpu",
    "summary": "python3 bench.py --summarize-kt rocprof_out/bench",
}
CALIB_BYTES = 64 * 2**20 * 4  # torch.neg over 64 Mi fp32: reads and writes this many bytes


def step_algo_bytes() -> int:
    """Bytes the fused step must move: the packed twin matrix, both x vectors,
    both y vectors, the two guess tokens, the two argmaxes and the accept count."""
    return ROWS * (COLS // 32) * 68 + 2 * COLS * 4 + 2 * ROWS * 4 + 2 * 4 + 2 * 4 + 4


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _csv_rows(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0], newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    """Kernel name without the parameter list (template arguments kept)."""
    name = name.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def summarize_kt(kt_dir, out_dir):
    """The kernel-trace statistics of the default bench run (every kernel it
    launches, mixed shapes per kernel name) as a text table under profiles/."""
    kt = _csv_rows(kt_dir, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel-trace statistics of the default bench.py run on one MI355X.  A kernel's row",
             "# mixes every shape that kernel ran; the headline step's GEMV (" + STEP_KERNEL + ") and",
             "# verify_keys_kernel run only in the step.  Per-call figures of single kernels are in the",
             "# gemv_*_isolated.txt profiles.",
             "", "command: " + KT_CMDS["kt"], "summary: " + KT_CMDS["summary"],
             "kernel_source_sha256: " + kernel_source_hash(), "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in kt:
        name = _short(r["Name"])
        name = name if len(name) <= 100 else name[:97] + "..."
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.2f} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, os.path.basename(KT_FILE)), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_kt_avg(kernel):
    """Average duration (us) of `kernel` in the committed default-run kernel-trace
    summary, or None if it is missing or the kernel source changed."""
    try:
        avg, src = None, None
        with open(KT_FILE) as f:
            for line in f:
                if line.startswith("kernel_source_sha256:"):
                    src = line.split(":", 1)[1].strip()
                elif line.startswith("| "):
                    cells = [c.strip() for c in line.strip().strip("|").split("|")]
                    if cells[0].endswith(kernel):
                        avg = float(cells[2])
        return avg if src == kernel_source_hash() else None
    except (OSError, ValueError, IndexError):
        return None


# Calls that can be launched alone for a per-kernel profile: name -> (what,
# kernel name as rocprofv3 reports it, format, streams).  At 17408 x 5120 one
# and two Q8 streams take the row-split kernel, four the per-wave-row kernel.
ISOLATED = {
    "ssq": ("SSQ twin GEMV alone (pti_gemv_ssq)", "gemv_ssq_split_kernel<5, 2, false, 8>", "ssq", 2),
    "step": ("fused SSQ twin GEMV + greedy verify (pti_gemv_ssq_verify)", "gemv_ssq_split_kernel<5, 2, true, 8>",
             "ssq", 2),
    "q8n1": ("Q8 GEMV, N = 1 (pti_gemv_q8_multi)", "gemv_q8_split_kernel<5, 1>", "q8", 1),
    "q8n2": ("Q8 GEMV, N = 2 (pti_gemv_q8_multi)", "gemv_q8_split_kernel<5, 2>", "q8", 2),
    "q8n4": ("Q8 GEMV, N = 4 (pti_gemv_q8_multi)", "gemv_kernel<0, 4, 4, 2, true, 16, 1, 0>", "q8", 4),
    # attention: format "attn", the last field the context length
    "attn4k": ("twin-KV decode attention (pti_attn_decode), 2 streams, 40 query heads over 8 kv heads of 128, "
               "4096 positions", "attn_partial_kernel<128, 5>", "attn", 4096),
    "attn32k": ("twin-KV decode attention (pti_attn_decode), 2 streams, 40 query heads over 8 kv heads of 128, "
                "32768 positions", "attn_partial_kernel<128, 5>", "attn", 32768),
}
ATTN_SHAPE = (2, 40, 8, 128)  # streams, query heads, kv heads, head dim
ATTN_COMBINE = "attn_combine_kernel<128>"

ISOLATED_CALLS = 60
SQ_COUNTERS = ("SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
               "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT")


def isolated_cmds(name):
    base = f"python3 bench.py --only {name} --no-cpu --copy-calibration"
    d = f"rocprof_out/{name}"
    return {
        "kt": f"rocprofv3 --kernel-trace --stats -f csv -d {d}/kt -o kt -- {base}",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE -f csv -d {d}/fetch -o fetch -- {base}",
        "write": f"rocprofv3 --pmc WRITE_SIZE TCC_HIT_sum TCC_MISS_sum -f csv -d {d}/write -o write -- {base}",
        "sq": f"rocprofv3 --pmc {' '.join(SQ_COUNTERS)} GRBM_GUI_ACTIVE -f csv -d {d}/sq -o sq -- {base}",
        "summary": f"python3 bench.py --summarize-isolated {name} {d}/kt {d}/fetch {d}/write {d}/write {d}/sq",
    }


def isolated_profile_path(name):
    _, _, fmt, n = ISOLATED[name]
    if fmt == "attn":
        return os.path.join(HERE, "profiles", f"attn_twin_h40_kv8_d128_ctx{n}_isolated.txt")
    return os.path.join(HERE, "profiles", f"gemv_{name}_17408x5120_isolated.txt")


def isolated_sources(name):
    return ATTN_SOURCES if ISOLATED[name][2] == "attn" else KERNEL_SOURCES


def isolated_run(torch, pti, dev, stream, name, calibrate):
    """ISOLATED_CALLS launches of one call over 17408 x 5120 (weights rotated over
    copies past the Infinity Cache), after the calibration copies if asked."""
    import synth
    L, sp = pti.lib(), pti._stream(stream)
    what, kernel, fmt, n = ISOLATED[name]
    if calibrate:
        src = torch.ones(64 * 2**20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if fmt == "attn":
        attn_isolated_run(torch, pti, dev, stream, name)
        return
    if fmt == "ssq":
        d = synth.twin(ROWS, COLS, synth.SEED_SSQ_FFN)
        P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
        X = np.stack([d["xA"], d["xB"]])
    else:
        d = synth.q8(ROWS, COLS, n, synth.SEED_Q8_FFN)
        P = pti.pack_q8(d["Q"], d["S"])
        X = d["X"]
    nc = copies_for(P.nbytes)
    w0 = torch.from_numpy(P).to(dev)
    ws = [w0] + [w0.clone() for _ in range(nc - 1)]
    x = torch.from_numpy(np.ascontiguousarray(X)).to(dev)
    y = torch.empty((max(n, 2), ROWS), dtype=torch.float32, device=dev)
    tok = torch.zeros(2, dtype=torch.int32, device=dev)
    am = torch.empty(2, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    work = pti.ssq_verify_workspace(dev)
    for i in range(ISOLATED_CALLS):
        w = ws[i % nc].data_ptr()
        if name == "ssq":
            st = L.pti_gemv_ssq(w, x[0].data_ptr(), x[1].data_ptr(), y[0].data_ptr(), y[1].data_ptr(), ROWS, COLS, sp)
        elif name == "step":
            st = L.pti_gemv_ssq_verify(w, x[0].data_ptr(), x[1].data_ptr(), y[0].data_ptr(), y[1].data_ptr(), ROWS,
                                       COLS, tok.data_ptr(), am.data_ptr(), acc.data_ptr(), work.data_ptr(),
                                       work.numel(), sp)
        else:
            st = L.pti_gemv_q8_multi(w, x.data_ptr(), y.data_ptr(), ROWS, COLS, n, sp)
        pti._check(name, st)
    torch.cuda.synchronize()
    log(f"isolated {name}: {ISOLATED_CALLS} launches of {what}, {nc} weight copies of {P.nbytes} B")


def attn_algo_bytes(L):
    """Algorithmic bytes of one attention call at the benchmark's shape with
    positions L - 2 and L - 1: the K and V rows 0..pos of both streams, q,
    k_new, v_new and out."""
    S, H, Hkv, d = ATTN_SHAPE
    kv_bytes = 2 * Hkv * d * 2 * ((L - 1) + L)
    return kv_bytes + 2 * S * H * d * 4 + 2 * S * Hkv * d * 4


def attn_isolated_run(torch, pti, dev, stream, name):
    """ISOLATED_CALLS attention calls at the benchmark's shape through the C
    entry point, caches rotated over sets of at least 640 MB in all."""
    what, _, _, L = ISOLATED[name]
    S, H, Hkv, d = ATTN_SHAPE
    set_bytes = 2 * S * Hkv * L * d * 2
    n_sets = max(2, -(-640 * 2**20 // set_bytes))
    kc = [[torch.randn((Hkv, L, d), device=dev).half() for _ in range(S)] for _ in range(n_sets)]
    vc = [[torch.randn((Hkv, L, d), device=dev).half() for _ in range(S)] for _ in range(n_sets)]
    q = torch.randn((S, H, d), device=dev)
    kn = torch.randn((S, Hkv, d), device=dev)
    vn = torch.randn((S, Hkv, d), device=dev)
    pos = torch.tensor([L - 2, L - 1], dtype=torch.int32, device=dev)
    work = pti.attn_workspace(S, H, Hkv, d, L, dev)
    o = torch.empty_like(q)
    lib, sp = pti.lib(), pti._stream(stream)
    ptrs = [((ctypes.c_void_p * S)(*[t.data_ptr() for t in kc[j]]),
             (ctypes.c_void_p * S)(*[t.data_ptr() for t in vc[j]])) for j in range(n_sets)]
    for i in range(ISOLATED_CALLS):
        kp, vp = ptrs[i % n_sets]
        pti._check(name, lib.pti_attn_decode(q.data_ptr(), kn.data_ptr(), vn.data_ptr(), kp, vp, pos.data_ptr(),
                                             o.data_ptr(), S, H, Hkv, d, L, work.data_ptr(), work.numel(), sp))
    torch.cuda.synchronize()
    log(f"isolated {name}: {ISOLATED_CALLS} calls of {what}, {n_sets} cache sets of {set_bytes} B")


def isolated_algo_bytes(name):
    _, _, fmt, n = ISOLATED[name]
    if fmt == "attn":
        return attn_algo_bytes(n)
    w = ROWS * (COLS // 32) * (68 if fmt == "ssq" else 34)
    extra = 20 if name == "step" else 0  # guess tokens, argmaxes, accept count
    return w + n * (COLS + ROWS) * 4 + extra


def summarize_isolated(name, kt_dir, fetch_dir, write_dir, tcc_dir, sq_dir, out_dir):
    """One call's profile from its --only runs: per-launch kernel time from the
    trace (for the fused step, also the span from the GEMV's start to the
    verify kernel's end; for attention, pass 2's time and the span from pass
    1's start to pass 2's end), HBM traffic (FETCH_SIZE, WRITE_SIZE scaled by
    the counters' reading for torch.neg over 256 MiB in the same run; for
    attention both passes), the L2 hit rate, and SQ counters (of the GEMV, or
    of attention's pass 1)."""
    what, kernel, fmt, n = ISOLATED[name]
    cmds = isolated_cmds(name)
    trace = _csv_rows(kt_dir, "kernel_trace.csv")
    disp = [r for r in trace if _short(r["Kernel_Name"]).endswith(kernel)]
    if len(disp) != ISOLATED_CALLS:
        raise SystemExit(f"{name}: expected {ISOLATED_CALLS} dispatches of {kernel}, found {len(disp)}")
    dur = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in disp[10:])
    med = dur[len(dur) // 2]
    avg = sum(dur) / len(dur)
    span = None
    second = {"step": "verify_keys_kernel"}.get(name, ATTN_COMBINE if fmt == "attn" else None)
    second_dur = None
    if second:
        # the call: the first kernel's start to the second one's end, dispatch by dispatch
        rows = sorted(trace, key=lambda r: int(r["Start_Timestamp"]))
        spans = []
        for i, r in enumerate(rows):
            if _short(r["Kernel_Name"]).endswith(kernel) and i + 1 < len(rows) and \
                    _short(rows[i + 1]["Kernel_Name"]).endswith(second):
                spans.append((int(rows[i + 1]["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        spans = sorted(spans[10:])
        span = (spans[len(spans) // 2], sum(spans) / len(spans))
        d2 = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                    for r in trace if _short(r["Kernel_Name"]).endswith(second))[10:]
        second_dur = d2[len(d2) // 2]

    def per_kernel(d, counter):
        acc = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] == counter:
                acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return acc

    def kern_avg(acc, key):
        ks = [k for k in acc if key(k)]
        if len(ks) != 1:
            raise SystemExit(f"{name}: expected one kernel, found {ks}")
        v = acc[ks[0]]
        return sum(v) / len(v), len(v)

    algo = isolated_algo_bytes(name)
    traffic = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        acc = per_kernel(d, counter)
        k_kib, k_n = kern_avg(acc, lambda k: k.endswith(kernel))
        if fmt == "attn":  # the call's traffic: both passes
            k_kib += kern_avg(acc, lambda k: k.endswith(ATTN_COMBINE))[0]
        c_kib, _ = kern_avg(acc, lambda k: "neg" in k.lower())
        factor = CALIB_BYTES / 1024.0 / c_kib
        traffic[counter] = (k_kib, k_n, factor, int(round(k_kib * 1024 * factor)))
    hits = per_kernel(tcc_dir, "TCC_HIT_sum")
    miss = per_kernel(tcc_dir, "TCC_MISS_sum")
    h, _ = kern_avg(hits, lambda k: k.endswith(kernel))
    m, _ = kern_avg(miss, lambda k: k.endswith(kernel))
    sq = {}
    for c in SQ_COUNTERS + ("GRBM_GUI_ACTIVE",):
        sq[c] = kern_avg(per_kernel(sq_dir, c), lambda k: k.endswith(kernel))[0]
    fb, wb = traffic["FETCH_SIZE"][3], traffic["WRITE_SIZE"][3]
    where = ("caches rotated over sets past the 256 MB Infinity Cache" if fmt == "attn" else
             "17408x5120, weights rotated over copies past the 256 MB Infinity Cache")
    lines = [f"# Isolated profile: {what}, one MI355X.",
             f"# {ISOLATED_CALLS} launches, {where}; durations",
             "# are per dispatch from the kernel trace (the first 10 dispatches left out); FETCH_SIZE and WRITE_SIZE",
             "# are scaled by their reading for torch.neg over 256 MiB (reads and writes 256 MiB) in the same run.",
             ""] + [f"command_{k}: {v}" for k, v in cmds.items()] + [
             "kernel_source_sha256: " + kernel_source_hash(isolated_sources(name)), "",
             f"kernel: {kernel}",
             f"dispatches: {len(disp)}",
             f"duration_us_median: {med:.3f}", f"duration_us_mean: {avg:.3f}",
             f"duration_us_min: {dur[0]:.3f}", f"duration_us_max: {dur[-1]:.3f}"]
    if span:
        if second_dur is not None and fmt == "attn":
            lines.append(f"second_kernel: {second}  median {second_dur:.3f} us (includes its wait behind pass 1)")
        lines += [f"call_span_us_median: {span[0]:.3f}  ({kernel} start to {second} end)",
                  f"call_span_us_mean: {span[1]:.3f}"]
    lines += [f"algorithmic_bytes_per_launch: {algo}",
              f"algorithmic_GBps_at_median: {algo / (med * 1e-6) / 1e9:.1f}",
              f"frac_of_8TBps_at_median: {algo / (med * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f}"]
    if span and fmt == "attn":
        lines += [f"frac_of_8TBps_at_call_span: {algo / (span[0] * 1e-6) / 1e9 / HBM_PEAK_GBS:.4f}"]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        k_kib, k_n, factor, b = traffic[counter]
        lines.append(f"{counter.lower()}_kib_per_dispatch: {k_kib:.1f} (x {factor:.4f} calibration = {b} B)")
    lines += [f"fetch_bytes_per_launch: {fb}", f"write_bytes_per_launch: {wb}",
              f"traffic_bytes_per_launch: {fb + wb}", f"traffic_over_algorithmic: {(fb + wb) / algo:.4f}",
              f"l2_hits: {h:.0f}", f"l2_misses: {m:.0f}", f"l2_hit_rate: {h / max(h + m, 1):.4f}"]
    for c, v in sq.items():
        lines.append(f"{c.lower()}: {v:.0f}")
    # derived.  A wave64 VALU instruction occupies its SIMD for 4 cycles; the
    # chip has 256 CUs x 4 SIMDs at 2.4 GHz (nominal).  Per weight: lane
    # operations over the weights one launch reads.
    simd_cycles = 1024 * med * 1e-6 * 2.4e9
    if fmt != "attn":
        weights = ROWS * COLS * (2 if fmt == "ssq" else 1)
        lines.append(f"valu_lane_ops_per_weight: {sq['SQ_INSTS_VALU'] * 64 / weights:.3f}")
    lines += [f"valu_busy_frac: {sq['SQ_INSTS_VALU'] * 4 / simd_cycles:.4f}  (VALU issue cycles / SIMD cycles at "
              f"the median duration and 2.4 GHz)",
              f"lds_busy_frac: {sq['SQ_INSTS_LDS'] * 64 * 16 / (256 * 128 * med * 1e-6 * 2.4e9):.4f}  (upper bound: "
              f"16 B per lane per LDS instruction at 128 B per CU-cycle)",
              f"lds_insts_per_valu_inst: {sq['SQ_INSTS_LDS'] / max(sq['SQ_INSTS_VALU'], 1):.4f}"]
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, os.path.basename(isolated_profile_path(name)))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_isolated(name):
    """{field: value} of a committed isolated profile, or None if it is missing
    or the kernel source changed since it was taken."""
    try:
        kv = {}
        with open(isolated_profile_path(name)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash(isolated_sources(name)):
            return None
        return kv
    except OSError:
        return None


def isolated_roofline(name, algo_bytes, us):
    """roofline block of a per-kernel entry: this run's time against 8 TB/s, with
    the kernel's trace duration, HBM traffic and L2 hit rate from its committed
    isolated profile (null when that profile is missing or stale)."""
    kv = read_isolated(name) or {}
    out = {"bound": "hbm", "achieved": round(algo_bytes / (us * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(algo_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "algorithmic_bytes_per_launch": algo_bytes,
           "traffic": int(kv["traffic_bytes_per_launch"]) if kv else None,
           "fetch_bytes": int(kv["fetch_bytes_per_launch"]) if kv else None,
           "rocprof_median_us": float(kv["duration_us_median"]) if kv else None,
           "l2_hit_rate": float(kv["l2_hit_rate"]) if kv else None,
           "profile": os.path.relpath(isolated_profile_path(name), HERE)}
    if kv:
        out["valu_busy_frac"] = float(kv["valu_busy_frac"].split()[0])
        if "valu_lane_ops_per_weight" in kv:
            out["valu_lane_ops_per_weight"] = float(kv["valu_lane_ops_per_weight"])
        if "call_span_us_median" in kv:
            out["rocprof_call_span_us"] = float(kv["call_span_us_median"].split()[0])
    return out


def tiny_twin(torch, pti, dev, stream):
    """The tiny SSQ twin workload (256 x 512, seed 0): latency-bound, timed for
    completeness; its outputs go to the parity check of the CPU leg."""
    import synth
    d = synth.twin(256, 512, synth.SEED_TINY)
    w = torch.from_numpy(pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])).to(dev)
    xa, xb = torch.from_numpy(d["xA"]).to(dev), torch.from_numpy(d["xB"]).to(dev)
    y = torch.empty((2, 256), device=dev)
    L = pti.lib()
    make = lambda sp: lambda i: pti._check("pti_gemv_ssq", L.pti_gemv_ssq(
        w.data_ptr(), xa.data_ptr(), xb.data_ptr(), y[0].data_ptr(), y[1].data_ptr(), 256, 512, sp))
    st = timed_stats(torch, make(pti._stream(stream)), stream, reps=5, per_rep=200)
    st["graph_us"] = graph_us(torch, pti, make)
    torch.cuda.synchronize()
    GPU_OUT["config1"] = (y[0].cpu().numpy().copy(), y[1].cpu().numpy().copy())
    return {"ssq_twin_256x512": {**st, "weight_bytes": int(w.numel())}}


def layer_sweep(torch, pti, dev, stream):
    """Every decoder-layer matrix (q, k, v, o 5120 wide; gate, up 17408 x 5120;
    down 5120 x 17408) from the seeded generator (seed 4): SSQ with distinct
    twins, SSQ with A == B, and Q8 (twin A's matrix) at N = 1, 2, 4 streams.
    Each matrix rotates over copies totalling at least 512 MB, so every launch
    reads its weights from HBM."""
    import synth
    L, sp = pti.lib(), pti._stream(stream)
    out = {}
    for name, rows, cols in synth.LAYER_SHAPES:
        twins = {"ssq": synth.twin(rows, cols, synth.SEED_LAYER),
                 "ssq_same": synth.twin(rows, cols, synth.SEED_LAYER, same=True)}
        twins["q8"] = twins["ssq"]  # Q8 runs twin A's matrix
        for variant in ("ssq", "ssq_same", "q8"):
            d = twins[variant]
            if variant == "q8":
                P = pti.pack_q8(d["A"], d["sA"])
                X = np.stack([d["xA"], d["xB"], -d["xA"], 0.5 * d["xB"]])
            else:
                P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
                X = np.stack([d["xA"], d["xB"]])
            nc = copies_for(P.nbytes)
            w0 = torch.from_numpy(P).to(dev)
            ws = [w0] + [w0.clone() for _ in range(nc - 1)]
            x = torch.from_numpy(np.ascontiguousarray(X)).to(dev)
            y = torch.empty((4, rows), device=dev)
            for n in ((2,) if variant != "q8" else (1, 2, 4)):
                if variant == "q8":
                    make = lambda sp, n=n: lambda i: pti._check("pti_gemv_q8_multi", L.pti_gemv_q8_multi(
                        ws[i % nc].data_ptr(), x.data_ptr(), y.data_ptr(), rows, cols, n, sp))
                else:
                    make = lambda sp: lambda i: pti._check("pti_gemv_ssq", L.pti_gemv_ssq(
                        ws[i % nc].data_ptr(), x[0].data_ptr(), x[1].data_ptr(), y[0].data_ptr(), y[1].data_ptr(),
                        rows, cols, sp))
                st = timed_stats(torch, make(sp), stream, reps=5, per_rep=100, warmup=20)
                st["graph_us"] = graph_us(torch, pti, make)
                torch.cuda.synchronize()
                key = f"layer_{name}_{variant}" + (f"_n{n}" if variant == "q8" else "")
                GPU_OUT[key] = y[:n].cpu().numpy().copy()
                us = st["median_us"]
                algo = P.nbytes + n * (rows + cols) * 4
                gus = st["graph_us"]
                out[key] = {**st, "rows": rows, "cols": cols, "weight_bytes": int(P.nbytes), "rotated_copies": nc,
                            "weight_GBps": round(P.nbytes / (us * 1e-6) / 1e9, 1),
                            "frac_of_hbm_peak": round(algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "graph_frac_of_hbm_peak": round(algo / (gus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                            "outputs_per_s": round(n * rows / (us * 1e-6), 1)}
            del ws, w0
            torch.cuda.empty_cache()
        log(f"layer {name}: " + ", ".join(f"{k[len('layer_' + name) + 1:]} {v['median_us']} us"
                                          for k, v in out.items() if k.startswith(f"layer_{name}_")))
    return out


def _median_time(fn, reps=3):
    ts = []
    res = None
    for _ in range(reps):
        t0 = time.perf_counter()
        res = fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2], res


def _ratio(got, want, t):
    got = np.asarray(got, np.float64)
    return float(np.max(np.abs(got - want) / np.maximum(t, 1e-300)))


def oracle_per_config():
    """The oracle (scalar C, one host thread) on each configuration the GPU ran,
    the median of 3 runs (one run of the toy decode loop), with the largest
    |y_gpu - y_oracle| / T over every output the GPU produced for it."""
    import oracle
    import synth
    from oracle import scalar, toy
    res = {}
    if "config1" in GPU_OUT:
        d = synth.twin(256, 512, synth.SEED_TINY)
        P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
        t, (ya, yb, ta, tb) = _median_time(lambda: oracle.gemv_ssq(P, 256, 512, d["xA"], d["xB"]))
        tp, _ = _median_time(lambda: scalar.gemv_ssq(P.tobytes(), 256, 512, d["xA"], d["xB"]))
        ga, gb = GPU_OUT["config1"]
        res["config1_ssq_twin_256x512"] = {"oracle_s": round(t, 5), "pure_python_s": round(tp, 3),
                                           "parity_max_err_over_T": max(_ratio(ga, ya, ta), _ratio(gb, yb, tb))}
    if "config2" in GPU_OUT:
        d = synth.twin(ROWS, COLS, synth.SEED_SSQ_FFN)
        P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
        t, (ya, yb, ta, tb) = _median_time(lambda: oracle.gemv_ssq(P, ROWS, COLS, d["xA"], d["xB"]))
        ga, gb = GPU_OUT["config2"]
        res["config2_ssq_twin_17408x5120"] = {"oracle_s": round(t, 4),
                                              "parity_max_err_over_T": max(_ratio(ga, ya, ta), _ratio(gb, yb, tb))}
    if "config3_n4" in GPU_OUT:
        q = synth.q8(ROWS, COLS, 4, synth.SEED_Q8_FFN)
        P = oracle.pack_q8(q["Q"], q["S"])
        for n in (1, 2, 4):
            t, (y, tt) = _median_time(lambda n=n: oracle.gemv_q8(P, ROWS, COLS, q["X"][:n]))
            res[f"config3_q8_17408x5120_n{n}"] = {"oracle_s": round(t, 4), "parity_max_err_over_T": max(
                _ratio(GPU_OUT[f"config3_n{n}"][s], y[s], tt[s]) for s in range(n))}
    for name, rows, cols in synth.LAYER_SHAPES:
        if f"layer_{name}_ssq" not in GPU_OUT:
            continue
        entry = {}
        twins = {"ssq": synth.twin(rows, cols, synth.SEED_LAYER),
                 "ssq_same": synth.twin(rows, cols, synth.SEED_LAYER, same=True)}
        twins["q8"] = twins["ssq"]
        for variant in ("ssq", "ssq_same", "q8"):
            d = twins[variant]
            if variant == "q8":
                P = oracle.pack_q8(d["A"], d["sA"])
                X = np.stack([d["xA"], d["xB"], -d["xA"], 0.5 * d["xB"]])
                t, (y, tt) = _median_time(lambda: oracle.gemv_q8(P, rows, cols, X))
                r = max(_ratio(GPU_OUT[f"layer_{name}_q8_n{n}"][s], y[s], tt[s]) for n in (1, 2, 4) for s in range(n))
            else:
                P = oracle.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
                t, (ya, yb, ta, tb) = _median_time(lambda: oracle.gemv_ssq(P, rows, cols, d["xA"], d["xB"]))
                g = GPU_OUT[f"layer_{name}_{variant}"]
                r = max(_ratio(g[0], ya, ta), _ratio(g[1], yb, tb))
            entry[variant] = {"oracle_s": round(t, 4), "parity_max_err_over_T": r}
        res[f"config4_layer_{name}_{rows}x{cols}"] = {
            **entry, "parity_max_err_over_T": max(v["parity_max_err_over_T"] for v in entry.values())}
    if "config5_n4" in GPU_OUT:
        raw = synth.toy_weights(synth.SEED_TOY)
        t0 = time.perf_counter()
        model = toy.ToyModel(raw, 1e-6)
        t_build = time.perf_counter() - t0
        t0 = time.perf_counter()
        committed, accepts, passes = toy.systolic_decode(
            lambda k, s, i, tok: toy.argmax_first(model.logits([tok])[0]), 1, 4, 64)
        t_loop = time.perf_counter() - t0
        gpu = GPU_OUT["config5_n4"].tolist()
        agree = sum(int(a == b) for a, b in zip(gpu, committed))
        res["config5_toy_decode_q8_n4_64steps"] = {
            "oracle_model_build_s": round(t_build, 2), "oracle_loop_s": round(t_loop, 2),
            "oracle_passes": len(passes), "oracle_mean_accept": round(float(np.mean(accepts)), 3),
            "committed_tokens_equal_to_gpu": f"{agree}/{len(committed)}", "parity_max_err_over_T": None}
    log(f"oracle per config: {json.dumps(res)}")
    return res


def layer_and_graph(torch, pti, dev, stream):
    """A decoder layer's GEMVs at their real shapes (q, k, v, o, gate, up,
    down; random packed weights, valid f16 scales): seven separate launches,
    four grouped launches (q|k|v, o, gate|up, down), and the grouped launches
    replayed from a captured graph.  Then the toy decoder's forward pass (Q8,
    four streams), eager against its native graph."""
    import synth
    out = {}
    shapes = {name: (r, c) for name, r, c in synth.LAYER_SHAPES}

    def packed(rows, cols, block):
        w = torch.randint(0, 256, (rows, cols // 32, block), dtype=torch.uint8, device=dev)
        w[:, :, 0] = 0x00
        w[:, :, 1] = 0x20  # f16 2^-7 in every scale slot
        if block == 68:
            w[:, :, 2] = 0x00
            w[:, :, 3] = 0x20
        return w.view(rows, -1)

    for fmt, block in (("q8", 34), ("ssq", 68)):
        W = {k: packed(*shapes[k], block) for k in shapes}
        wbytes = sum(t.numel() for t in W.values())
        for n in ((1, 4) if fmt == "q8" else (2,)):
            x5 = torch.randn((n, 5120), device=dev)
            x17 = torch.randn((n, 17408), device=dev)
            y = {k: torch.empty((n, shapes[k][0]), device=dev) for k in shapes}
            yqkv = torch.empty((n, 7168), device=dev)
            ygu = torch.empty((n, 34816), device=dev)
            if fmt == "q8":
                # launches go to the current stream: the bench stream, or the
                # capture stream inside torch.cuda.graph
                def one(k, x):
                    pti.gemv_q8_multi(W[k], x, y[k])

                def grp(ks, x, yy):
                    pti.gemv_q8_multi_grouped([W[k] for k in ks], x, yy)
            else:
                def one(k, x):
                    pti.gemv_ssq(W[k], x[0], x[1], y[k][0], y[k][1])

                def grp(ks, x, yy):
                    pti.gemv_ssq_grouped([W[k] for k in ks], x[0], x[1], yy[0], yy[1])

            def separate(i):
                for k in ("q", "k", "v", "o", "gate", "up"):
                    one(k, x5)
                one("down", x17)

            def grouped(i):
                grp(("q", "k", "v"), x5, yqkv)
                one("o", x5)
                grp(("gate", "up"), x5, ygu)
                one("down", x17)

            st_sep = timed_stats(torch, separate, stream, reps=5, per_rep=50, warmup=10)
            st_grp = timed_stats(torch, grouped, stream, reps=5, per_rep=50, warmup=10)
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                grouped(0)
            st_graph = timed_stats(torch, lambda i: g.replay(), stream, reps=5, per_rep=50, warmup=10)
            key = f"layer_{fmt}_n{n}"
            out[key] = {"weight_bytes": wbytes, "separate_us": st_sep["median_us"], "grouped_us": st_grp["median_us"],
                        "graph_us": st_graph["median_us"],
                        "graph_weight_GBps": round(wbytes / (st_graph["median_us"] * 1e-6) / 1e9, 1)}
            log(f"{key}: {out[key]}")
            del g
        del W
        torch.cuda.empty_cache()

    # toy decoder forward pass (hidden 2048, ffn 5632, 4 layers, vocab 32000), Q8, N = 4
    raw = synth.toy_weights(synth.SEED_TOY)
    q = lambda m: torch.from_numpy(pti.pack_q8(m["Q"], m["S"])).to(dev)
    mats = {"emb": q(raw["emb"]), "head": q(raw["head"]), "gate": [q(l["gate"]) for l in raw["layers"]],
            "up": [q(l["up"]) for l in raw["layers"]], "down": [q(l["down"]) for l in raw["layers"]]}
    stack = pti.ToyStack(mats, 2048, 5632, 32000, pti.FMT_Q8, 1e-6)
    toks = torch.tensor([1, 2, 3, 4], dtype=torch.int32, device=dev)
    logits = torch.empty((4, 32000), device=dev)
    work = stack.workspace(4)
    st_eager = timed_stats(torch, lambda i: stack.forward(toks, logits, work, stream=stream), stream, reps=5,
                           per_rep=50, warmup=10)
    graph = stack.forward_graph(toks, logits, work)
    st_g = timed_stats(torch, lambda i: graph.launch(stream=stream), stream, reps=5, per_rep=50, warmup=10)
    graph.destroy()
    wbytes = sum(t.numel() for t in [mats["head"]] + mats["gate"] + mats["up"] + mats["down"])
    out["toy_forward_q8_n4"] = {"eager_us": st_eager["median_us"], "graph_us": st_g["median_us"],
                                "gemv_weight_bytes": wbytes,
                                "graph_weight_GBps": round(wbytes / (st_g["median_us"] * 1e-6) / 1e9, 1)}
    log(f"toy forward: {out['toy_forward_q8_n4']}")

    # the staggered twin-decode loop itself (greedy, 64 steps, the host reads
    # each step's draws back), N = 1 and N = 4 streams
    for n in (1, 4):
        w_n = stack.workspace(n)
        stack.decode(1, n, 4, work=w_n)  # warm-up
        torch.cuda.synchronize()
        reps = []
        for _ in range(5):
            t0 = time.perf_counter()
            committed, accepts, passes = stack.decode(1, n, 64, work=w_n)
            reps.append(time.perf_counter() - t0)
        t = sorted(reps)[2]
        # passes rows are (step, slot, stream, input, output): an N-stream pass
        # has slots 0..N-1, a single-stream (ramp-up or redraw) pass a slot >= N
        fwd = 64 + int((passes[:, 1] >= n).sum()) if n > 1 else 64
        GPU_OUT[f"config5_n{n}"] = np.asarray(committed).copy()
        out[f"toy_decode_q8_n{n}_64steps"] = {
            "ms": round(t * 1e3, 3), "forward_passes": fwd, "us_per_step": round(t / 64 * 1e6, 2),
            "us_per_forward_pass": round(t / fwd * 1e6, 2),
            "steps_per_s": round(64 / t, 1),  # one committed token per step (stream 0's draw)
            "mean_accept": round(float(accepts.mean()), 3)}  # the pages' tokens per step, 1 + p + p^2 + ...
        log(f"toy decode n={n}: {out[f'toy_decode_q8_n{n}_64steps']}")
    return out


def verify_and_pack(torch, pti, dev, stream, d):
    """The verify calls at the toy decoder's vocabulary (32000) for N = 1, 2, 4
    streams, greedy and sampled (temperature 0.7), time per call; and the host
    packer over the 17408x5120 twin (one call, median of three)."""
    out = {}
    L, sp = pti.lib(), pti._stream(stream)
    g = torch.Generator(device="cpu").manual_seed(5)
    for n in (1, 2, 4):
        logits = torch.randn((n, 32000), generator=g).to(dev)
        tok = torch.zeros(n, dtype=torch.int32, device=dev)
        am = torch.empty(n, dtype=torch.int32, device=dev)
        acc = torch.empty(1, dtype=torch.int32, device=dev)
        make = lambda sp: lambda i: L.pti_verify_argmax(logits.data_ptr(), tok.data_ptr(), am.data_ptr(),
                                                        acc.data_ptr(), 32000, n, sp)
        st = timed_stats(torch, make(sp), stream, reps=5, per_rep=50, warmup=10)
        st["graph_us"] = graph_us(torch, pti, make)
        out[f"verify_greedy_n{n}_v32000"] = st
        u = torch.rand(n, dtype=torch.float64, generator=g).to(dev)
        sw = pti.sample_verify_workspace(32000, n, dev)
        make = lambda sp: lambda i: L.pti_sample_verify(logits.data_ptr(), tok.data_ptr(), u.data_ptr(), 0.7,
                                                        am.data_ptr(), acc.data_ptr(), 32000, n, sw.data_ptr(),
                                                        sw.numel(), sp)
        st = timed_stats(torch, make(sp), stream, reps=5, per_rep=50, warmup=10)
        st["graph_us"] = graph_us(torch, pti, make)
        out[f"verify_sampled_n{n}_v32000_t0.7"] = st
        log(f"verify n={n}: {out[f'verify_greedy_n{n}_v32000']}")
    ts = []
    for _ in range(3):
        t0 = time.perf_counter()
        P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
        ts.append(time.perf_counter() - t0)
    t = sorted(ts)[1]
    # the packer splits rows over std::thread workers: the host's hardware threads, at most 32
    out["host_pack_ssq_17408x5120"] = {"ms": round(t * 1e3, 3), "out_bytes": int(P.nbytes),
                                       "out_GBps": round(P.nbytes / t / 1e9, 3),
                                       "threads": min(os.cpu_count() or 1, 32)}
    log(f"host pack: {out['host_pack_ssq_17408x5120']}")
    return out


def attention(torch, pti, dev, stream):
    """Twin-KV decode attention (two streams: the twins), 40 query heads over
    8 kv heads of 128, binary16 caches, at 4K and 32K positions: time per
    call and the K/V bytes it must read against 8 TB/s.  Successive calls
    rotate over enough cache sets (at least 640 MB in all) that a call's
    cache rows are not still in the 256 MB Infinity Cache from an earlier
    call."""
    out = {}
    S, H, Hkv, d = 2, 40, 8, 128
    for L in (4096, 32768):
        set_bytes = 2 * S * Hkv * L * d * 2
        n_sets = max(2, -(-640 * 2**20 // set_bytes))
        kc = [[torch.randn((Hkv, L, d), device=dev).half() for _ in range(S)] for _ in range(n_sets)]
        vc = [[torch.randn((Hkv, L, d), device=dev).half() for _ in range(S)] for _ in range(n_sets)]
        q = torch.randn((S, H, d), device=dev)
        kn = torch.randn((S, Hkv, d), device=dev)
        vn = torch.randn((S, Hkv, d), device=dev)
        pos = torch.tensor([L - 2, L - 1], dtype=torch.int32, device=dev)
        work = pti.attn_workspace(S, H, Hkv, d, L, dev)
        o = torch.empty_like(q)
        # the C entry point with pointer arrays built once per cache set (the
        # binding's per-call checks would make a 4K call host-bound)
        lib, sp = pti.lib(), pti._stream(stream)
        ptrs = [((ctypes.c_void_p * S)(*[t.data_ptr() for t in kc[j]]),
                 (ctypes.c_void_p * S)(*[t.data_ptr() for t in vc[j]])) for j in range(n_sets)]

        args = (q.data_ptr(), kn.data_ptr(), vn.data_ptr(), pos.data_ptr(), o.data_ptr(), work.data_ptr(),
                work.numel())

        def make(sp, a=args):
            def call(i):
                kp, vp = ptrs[i % n_sets]
                st = lib.pti_attn_decode(a[0], a[1], a[2], kp, vp, a[3], a[4], S, H, Hkv, d, L, a[5], a[6], sp)
                if st:
                    pti._check("pti_attn_decode", st)
            return call
        st = timed_stats(torch, make(sp), stream, reps=5, per_rep=50, warmup=10)
        st["graph_us"] = graph_us(torch, pti, make)
        kv_bytes = 2 * Hkv * d * 2 * ((L - 1) + L)  # K and V rows 0..pos of both streams
        algo = kv_bytes + 2 * S * H * d * 4 + 2 * S * Hkv * d * 4
        out[f"attn_twin_h40_kv8_d128_ctx{L}"] = {
            **st, "kv_bytes": kv_bytes, "algorithmic_bytes": algo, "cache_sets": n_sets,
            "roofline": isolated_roofline("attn4k" if L == 4096 else "attn32k", algo, st["median_us"]),
            "GBps": round(algo / (st["median_us"] * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(algo / (st["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "graph_frac_of_hbm_peak": round(algo / (st["graph_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"attention ctx {L}: {out[f'attn_twin_h40_kv8_d128_ctx{L}']}")
        del kc, vc, work
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-main", action="store_true",
                    help="time the fused SSQ step only, no other kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --only: first run 3 elementwise copies of 256 MiB (reference kernel for HBM byte "
                         "counters)")
    ap.add_argument("--summarize-kt", metavar="KT_DIR",
                    help="write the default run's kernel-trace summary from rocprofv3 CSV output (CPU only) and exit")
    ap.add_argument("--profiles-out", default=os.path.join(HERE, "profiles"))
    ap.add_argument("--only", choices=sorted(ISOLATED),
                    help="launch only this call (a few times, weights rotated) and exit: the runs behind the "
                         "per-kernel profiles")
    ap.add_argument("--summarize-isolated", nargs=6, metavar=("NAME", "KT_DIR", "FETCH_DIR", "WRITE_DIR", "TCC_DIR",
                                                              "SQ_DIR"),
                    help="write profiles/<summary of NAME> from the rocprofv3 output of its --only runs (CPU only)")
    args = ap.parse_args()
    if args.summarize_isolated:
        summarize_isolated(*args.summarize_isolated, args.profiles_out)
        return
    if args.summarize_kt:
        summarize_kt(args.summarize_kt, args.profiles_out)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import packed_twin_int8_amd as pti
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    log(f"device {torch.cuda.get_device_name(0)}")
    if args.only:
        isolated_run(torch, pti, dev, stream, args.only, args.copy_calibration)
        return

    # ---------------- inputs: SSQ twin workload, seed 2
    d = synth.twin(ROWS, COLS, synth.SEED_SSQ_FFN)
    P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    w_bytes = P.nbytes
    n_copies = copies_for(w_bytes)
    w0 = torch.from_numpy(P).to(dev)
    ws = [w0] + [w0.clone() for _ in range(n_copies - 1)]
    xa = torch.from_numpy(d["xA"]).to(dev)
    xb = torch.from_numpy(d["xB"]).to(dev)
    ya = torch.empty(ROWS, dtype=torch.float32, device=dev)
    yb = torch.empty(ROWS, dtype=torch.float32, device=dev)
    y2 = torch.stack([ya, yb])  # verify reads [2][ROWS]; GEMV writes into its rows
    ya, yb = y2[0], y2[1]
    tok = torch.zeros(2, dtype=torch.int32, device=dev)
    am = torch.empty(2, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    work = pti.ssq_verify_workspace(dev)
    L = pti.lib()
    sp = pti._stream(stream)

    def gemv(i):
        st = L.pti_gemv_ssq(ws[i % n_copies].data_ptr(), xa.data_ptr(), xb.data_ptr(), ya.data_ptr(), yb.data_ptr(),
                            ROWS, COLS, sp)
        if st:
            pti._check("pti_gemv_ssq", st)

    def verify(i):
        st = L.pti_verify_argmax(y2.data_ptr(), tok.data_ptr(), am.data_ptr(), acc.data_ptr(), ROWS, 2, sp)
        if st:
            pti._check("pti_verify_argmax", st)

    def step(i):
        st = L.pti_gemv_ssq_verify(ws[i % n_copies].data_ptr(), xa.data_ptr(), xb.data_ptr(), ya.data_ptr(),
                                   yb.data_ptr(), ROWS, COLS, tok.data_ptr(), am.data_ptr(), acc.data_ptr(),
                                   work.data_ptr(), work.numel(), sp)
        if st:
            pti._check("pti_gemv_ssq_verify", st)

    log(f"ssq twin {ROWS}x{COLS}: {w_bytes} weight bytes, {n_copies} copies rotated")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms_step = timed_loop(torch, step, args.steps, stream)
    log(f"step: {ms_step * 1e3:.2f} us")

    algo_bytes = step_algo_bytes()
    assert algo_bytes - w_bytes == 2 * COLS * 4 + 2 * ROWS * 4 + 20
    st_fused = timed_stats(torch, step, stream)
    ms_fused = st_fused["median_us"] * 1e-3
    log(f"fused gemv+verify: {st_fused}")
    torch.cuda.synchronize()
    GPU_OUT["config2"] = (ya.cpu().numpy().copy(), yb.cpu().numpy().copy())
    per_kernel = {}
    copy_GBps = None
    if not args.only_main:
        st_gemv = timed_stats(torch, gemv, stream)
        st_verify = timed_stats(torch, verify, stream)
        ms_gemv = st_gemv["median_us"] * 1e-3
        log(f"unfused: ssq gemv alone {st_gemv}; verify alone {st_verify}")
        per_kernel["ssq_twin_gemv_unfused"] = {**st_gemv,
                                               "weight_GBps": round(w_bytes / (ms_gemv * 1e-3) / 1e9, 2),
                                               "roofline": isolated_roofline("ssq", isolated_algo_bytes("ssq"),
                                                                             st_gemv["median_us"])}
        per_kernel["verify_n2_v17408_unfused"] = st_verify
        # two streams per twin: four activation vectors per weight read
        xa2 = torch.randn((2, COLS), device=dev)
        xb2 = torch.randn((2, COLS), device=dev)
        ya2 = torch.empty((2, ROWS), device=dev)
        yb2 = torch.empty((2, ROWS), device=dev)

        def gemv2(i):
            st = L.pti_gemv_ssq_multi(ws[i % n_copies].data_ptr(), xa2.data_ptr(), xb2.data_ptr(), ya2.data_ptr(),
                                      yb2.data_ptr(), ROWS, COLS, 2, sp)
            if st:
                pti._check("pti_gemv_ssq_multi", st)
        st_g2 = timed_stats(torch, gemv2, stream)
        per_kernel["ssq_gemv_2_per_twin"] = {
            **st_g2, "weight_GBps": round(w_bytes / (st_g2["median_us"] * 1e-6) / 1e9, 2),
            "outputs_per_s": round(4 * ROWS / (st_g2["median_us"] * 1e-6), 1),
            "cost_over_1_per_twin": round(st_g2["median_us"] / st_gemv["median_us"], 4)}
        log(f"ssq 2 per twin: {st_g2}")
        # device-to-device copy of the same byte count, rotated the same way:
        # the practical ceiling (reads and writes w_bytes each)
        dsts = [torch.empty_like(w0) for _ in range(2)]
        st_copy = timed_stats(torch, lambda i: dsts[i % 2].copy_(ws[i % n_copies]), stream)
        copy_GBps = 2 * w_bytes / (st_copy["median_us"] * 1e-6) / 1e9
        del dsts
        log(f"copy {w_bytes} B: {st_copy}, {copy_GBps:.0f} GB/s read+write")

    prof = read_isolated("step") or {}
    result = {
        "metric": METRIC,
        "value": round(w_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "ssq_twin_gemv_17408x5120+greedy_verify (fused)",
            "rows": ROWS, "cols": COLS, "format": "SSQ mode-16 (68 B blocks), int8 twins, f16 block scales",
            "streams": 2, "seed": synth.SEED_SSQ_FFN, "weight_copies_rotated": n_copies,
            "rotated_bytes": n_copies * w_bytes, "device": torch.cuda.get_device_name(0),
        },
        "gemv_per_s": round(1.0 / (ms_step * 1e-3), 1),
        "frac_of_hbm_peak": round(w_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "pti_gemv_ssq_verify = gemv_ssq_split_kernel<5, 2, true, 8> + verify_keys_kernel",
            "achieved": round(algo_bytes / (ms_fused * 1e-3) / 1e9, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(algo_bytes / (ms_fused * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": int(prof["traffic_bytes_per_launch"]) if prof else None,
            "algorithmic_bytes_per_launch": algo_bytes,
            "avg_launch_us": round(ms_fused * 1e3, 3),
            "launch_us_stats": st_fused,
            "vs_copy": round(algo_bytes / (ms_fused * 1e-3) / 1e9 / copy_GBps, 4) if copy_GBps else None,
            # from the committed isolated profile of this call (null if missing or stale): the GEMV
            # kernel's trace duration, and the call's span from the GEMV's start to the verify
            # kernel's end, per dispatch, medians
            "rocprof_gemv_kernel_us": float(prof["duration_us_median"]) if prof else None,
            "rocprof_call_span_us": float(prof["call_span_us_median"].split()[0]) if prof else None,
            "rocprof_default_run_gemv_avg_us": read_kt_avg(STEP_KERNEL),
            "l2_hit_rate": float(prof["l2_hit_rate"]) if prof else None,
            "profile": os.path.relpath(isolated_profile_path("step"), HERE),
            "kernel_stats": os.path.relpath(KT_FILE, HERE),
        },
    }
    if copy_GBps:
        result["copy_ceiling"] = {"GBps_read_plus_write": round(copy_GBps, 1), "bytes_each_way": w_bytes, **st_copy}
    del ws, w0
    torch.cuda.empty_cache()

    # ---------------- Q8 multi-stream, N = 1, 2, 4
    if not args.only_main:
        q = synth.q8(ROWS, COLS, 4, synth.SEED_Q8_FFN)
        Pq = pti.pack_q8(q["Q"], q["S"])
        nq = copies_for(Pq.nbytes)
        wq0 = torch.from_numpy(Pq).to(dev)
        wqs = [wq0] + [wq0.clone() for _ in range(nq - 1)]
        X = torch.from_numpy(q["X"]).to(dev)
        Y = torch.empty((4, ROWS), dtype=torch.float32, device=dev)
        t = {}
        for n in (1, 2, 4):
            def qgemv(i, n=n):
                st = L.pti_gemv_q8_multi(wqs[i % nq].data_ptr(), X.data_ptr(), Y.data_ptr(), ROWS, COLS, n, sp)
                if st:
                    pti._check("pti_gemv_q8_multi", st)
            stn = timed_stats(torch, qgemv, stream)
            t[n] = stn["median_us"] * 1e-3
            algo = Pq.nbytes + n * (COLS + ROWS) * 4
            torch.cuda.synchronize()
            GPU_OUT[f"config3_n{n}"] = Y[:n].cpu().numpy().copy()
            per_kernel[f"q8_gemv_n{n}"] = {
                "us": round(t[n] * 1e3, 3), **stn,
                "weight_GBps": round(Pq.nbytes / (t[n] * 1e-3) / 1e9, 2),
                "frac_of_hbm_peak": round(algo / (t[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "gemv_per_s": round(1 / (t[n] * 1e-3), 1),
                "outputs_per_s": round(n * ROWS / (t[n] * 1e-3), 1),
                "roofline": isolated_roofline(f"q8n{n}", algo, t[n] * 1e3),
            }
            log(f"q8 n={n}: {t[n] * 1e3:.2f} us, {Pq.nbytes / (t[n] * 1e-3) / 1e9:.1f} GB/s")
        per_kernel["q8_step_cost_n4_over_n1"] = round(t[4] / t[1], 4)
        del wqs, wq0
        torch.cuda.empty_cache()
        per_kernel.update(tiny_twin(torch, pti, dev, stream))
        per_kernel.update(layer_sweep(torch, pti, dev, stream))
        per_kernel.update(layer_and_graph(torch, pti, dev, stream))
        per_kernel.update(attention(torch, pti, dev, stream))
        per_kernel.update(verify_and_pack(torch, pti, dev, stream, d))
    result["per_kernel"] = per_kernel

    if not args.no_cpu:
        log("cpu baseline (oracle)...")
        result["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
        if not args.only_main:
            result["cpu_baseline"]["per_config"] = oracle_per_config()
            result["parity_max_err_over_T"] = max(
                v["parity_max_err_over_T"] for v in result["cpu_baseline"]["per_config"].values()
                if v.get("parity_max_err_over_T") is not None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

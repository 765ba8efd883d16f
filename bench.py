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
TRAFFIC_FILE = os.path.join(HERE, "profiles", "gemv_ssq_verify_17408x5120_pmc.txt")
KT_FILE = os.path.join(HERE, "profiles", "gemv_ssq_q8_17408x5120_kernel_stats.md")
# the step's kernels, as rocprofv3 names them (template arguments kept)
STEP_KERNELS = ("gemv_ssq_split_kernel<5, 2, true, 8>", "verify_keys_kernel")
KERNEL_SOURCES = ("packed_twin_int8_amd/csrc/pti_gemv.hip", "packed_twin_int8_amd/build.py")
PROFILE_CMDS = {
    "kt": "rocprofv3 --kernel-trace --stats -f csv -d rocprof_out/kt -o kt -- python3 bench.py --no-cpu",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d rocprof_out/fetch -o fetch -- "
             "python3 bench.py --only-main --no-cpu --steps 10 --warmup 2 --copy-calibration",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d rocprof_out/write -o write -- "
             "python3 bench.py --only-main --no-cpu --steps 10 --warmup 2 --copy-calibration",
    "summary": "python3 bench.py --summarize-profiles rocprof_out/kt rocprof_out/fetch "
               "rocprof_out/write --profiles-out profiles",
    "tcc": "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum -f csv -d rocprof_out/tcc -o tcc -- "
           "python3 bench.py --cache-profile --no-cpu",
    "tcc_summary": "python3 bench.py --summarize-hit-rate rocprof_out/tcc --profiles-out profiles",
}
HIT_FILE = os.path.join(HERE, "profiles", "gemv_l2_hit_rate_17408x5120_pmc.txt")
# kernels of the cache-profile run, as rocprofv3 names them, and what each one is there
HIT_KERNELS = {
    "gemv_ssq_split_kernel<5, 2, true, 8>": "step: fused SSQ twin GEMV (+ verify keys)",
    "verify_keys_kernel": "step: verify keys",
    "gemv_ssq_split_kernel<5, 2, false, 8>": "SSQ twin GEMV alone",
    "gemv_q8_split_kernel<5, 1>": "Q8 GEMV, N = 1",
    "gemv_q8_split_kernel<5, 2>": "Q8 GEMV, N = 2",
    "gemv_kernel<0, 4, 4, 2, true, 16, 4>": "Q8 GEMV, N = 4",
}
# the Q8 kernel of each stream count at 17408 x 5120 (one and two streams take
# the row-split kernel there, four the per-wave-row kernel)
Q8_KERNEL = {1: "gemv_q8_split_kernel<5, 1>", 2: "gemv_q8_split_kernel<5, 2>", 4: "gemv_kernel<0, 4, 4, 2, true, 16, 4>"}
CALIB_BYTES = 64 * 2**20 * 4  # torch.neg over 64 Mi fp32: reads and writes this many bytes


def step_algo_bytes() -> int:
    """Bytes the fused step must move: the packed twin matrix, both x vectors,
    both y vectors, the two guess tokens, the two argmaxes and the accept count."""
    return ROWS * (COLS // 32) * 68 + 2 * COLS * 4 + 2 * ROWS * 4 + 2 * 4 + 2 * 4 + 4


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per SSQ GEMV launch from the committed PMC summary, or None if
    there is none or the kernel source changed since the counters were taken."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith((" ", "#", "|")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return {"bytes": int(kv["traffic_bytes_per_launch"]), "fetch_bytes": int(kv["fetch_bytes_per_launch"]),
                "write_bytes": int(kv["write_bytes_per_launch"]), "source": os.path.relpath(TRAFFIC_FILE, HERE)}
    except (OSError, KeyError, ValueError):
        return None


def read_kernel_avgs():
    """rocprofv3 average duration (us) of each step kernel from the committed
    kernel-trace summary, or None if it is missing or the source changed."""
    try:
        avgs, src = {}, None
        with open(KT_FILE) as f:
            for line in f:
                if line.startswith("kernel_source_sha256:"):
                    src = line.split(":", 1)[1].strip()
                elif line.startswith("| "):
                    cells = [c.strip() for c in line.strip().strip("|").split("|")]
                    for k in STEP_KERNELS:
                        if cells[0].endswith(k):
                            avgs[k] = float(cells[2])
        if src != kernel_source_hash() or len(avgs) != len(STEP_KERNELS):
            return None
        return avgs
    except (OSError, ValueError, IndexError):
        return None


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


def summarize_profiles(kt_dir, fetch_dir, write_dir, out_dir):
    """Turn rocprofv3 CSV output into the text summaries kept under profiles/."""
    src_hash = kernel_source_hash()
    kt = _csv_rows(kt_dir, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel-trace statistics: bench.py default run on one MI355X: the fused SSQ twin GEMV",
             "# 17408x5120 + verify (the step), the unfused GEMV and verify, SSQ with two streams per twin, Q8",
             "# multi-stream GEMV 17408x5120 at N=1,2,4, a decoder layer's GEMVs (separate, grouped, graph), the",
             "# toy decoder forward pass, and twin-KV attention at 4K and 32K positions.  A kernel's row mixes",
             "# every shape it ran; the step's kernels (gemv_ssq_split_kernel<5, 2, true, 8>, verify_keys_kernel)",
             "# run only in the step.",
             "", "command: " + PROFILE_CMDS["kt"], "summary: " + PROFILE_CMDS["summary"],
             "kernel_source_sha256: " + src_hash, "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in kt:
        name = _short(r["Name"])
        name = name if len(name) <= 100 else name[:97] + "..."
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.2f} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, "gemv_ssq_q8_17408x5120_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(d, counter):
        acc = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return acc

    def pick(acc, key):
        ks = [k for k in acc if key(k)]
        if len(ks) != 1:
            raise SystemExit(f"expected one kernel, found {ks}")
        v = acc[ks[0]]
        return ks[0], sum(v) / len(v), len(v)

    out = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        acc = per_kernel(d, counter)
        # the PMC runs launch only the step's kernels (and the calibration copy)
        steps = [pick(acc, lambda k, sk=sk: k.endswith(sk)) for sk in STEP_KERNELS]
        cname, c_kib, c_n = pick(acc, lambda k: "neg_kernel" in k or "neg" in k.lower())
        factor = CALIB_BYTES / 1024.0 / c_kib
        g_kib = sum(k for _, k, _ in steps)
        out[counter] = dict(steps=steps, g_kib=g_kib, cname=cname, c_kib=c_kib, c_n=c_n, factor=factor,
                            bytes=int(round(g_kib * 1024 * factor)))
    algo = step_algo_bytes()
    fb, wb = out["FETCH_SIZE"]["bytes"], out["WRITE_SIZE"]["bytes"]
    lines = ["# HBM traffic of the fused SSQ twin GEMV + verify (17408x5120; both kernels of one call),",
             "# rocprofv3 PMC counters, one MI355X",
             "# Each counter is scaled by the ratio of known bytes to the counter's reading for torch.neg",
             "# over 256 MiB (reads 256 MiB, writes 256 MiB) in the same run.",
             "", "command_fetch: " + PROFILE_CMDS["fetch"], "command_write: " + PROFILE_CMDS["write"],
             "summary: " + PROFILE_CMDS["summary"], ""]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[counter]
        lines += [f"| {counter} | kernel | dispatches | avg KiB/dispatch |", "|---|---|---|---|"]
        lines += [f"| | {n} | {cnt} | {kib:.1f} |" for n, kib, cnt in o["steps"]]
        lines += [f"| | step total | | {o['g_kib']:.1f} |",
                  f"| | {o['cname'][:90]} (calibration, {CALIB_BYTES} B) | {o['c_n']} | {o['c_kib']:.1f} |",
                  f"calibration factor {counter}: {o['factor']:.4f}", ""]
    lines += [f"algorithmic_bytes_per_launch: {algo}",
              f"fetch_bytes_per_launch: {fb}", f"write_bytes_per_launch: {wb}",
              f"traffic_bytes_per_launch: {fb + wb}",
              f"traffic_over_algorithmic: {(fb + wb) / algo:.4f}",
              "kernel_source_sha256: " + src_hash]
    with open(os.path.join(out_dir, os.path.basename(TRAFFIC_FILE)), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_hit_rate(tcc_dir, out_dir):
    """L2 (TCC) hit rate per kernel of the cache-profile run, from rocprofv3's
    TCC_HIT_sum and TCC_MISS_sum: the share of L2 requests served without a
    fetch from the Infinity Fabric (x re-reads hit; streamed weights miss)."""
    acc = {}
    for r in _csv_rows(tcc_dir, "counter_collection.csv"):
        k = _short(r["Kernel_Name"])
        acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# L2 (TCC) hit rate per kernel: the fused SSQ step, the SSQ GEMV alone and the Q8 GEMV at",
             "# N = 1, 2, 4 streams over 17408x5120 (weights rotated over copies larger than the Infinity Cache),",
             "# rocprofv3 PMC counters TCC_HIT_sum and TCC_MISS_sum, one MI355X.  hit rate = hits / (hits + misses).",
             "", "command: " + PROFILE_CMDS["tcc"], "summary: " + PROFILE_CMDS["tcc_summary"],
             "kernel_source_sha256: " + kernel_source_hash(), "",
             "| kernel | what | dispatches | avg hits | avg misses | hit rate |", "|---|---|---|---|---|---|"]
    found = 0
    for name, what in HIT_KERNELS.items():
        ks = [k for k in acc if k.endswith(name)]
        if len(ks) != 1:
            raise SystemExit(f"expected one kernel named {name}, found {ks}")
        c = acc[ks[0]]
        h, m = c.get("TCC_HIT_sum", []), c.get("TCC_MISS_sum", [])
        if not h or len(h) != len(m):
            raise SystemExit(f"{name}: missing TCC counters")
        hh, mm = sum(h) / len(h), sum(m) / len(m)
        lines.append(f"| {name} | {what} | {len(h)} | {hh:.0f} | {mm:.0f} | {hh / max(hh + mm, 1):.4f} |")
        found += 1
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, os.path.basename(HIT_FILE)), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_hit_rates():
    """{kernel: L2 hit rate} from the committed summary, or None if it is
    missing or the kernel source changed since the counters were taken."""
    try:
        rates, src = {}, None
        with open(HIT_FILE) as f:
            for line in f:
                if line.startswith("kernel_source_sha256:"):
                    src = line.split(":", 1)[1].strip()
                elif line.startswith("| ") and not line.startswith("| kernel"):
                    cells = [c.strip() for c in line.strip().strip("|").split("|")]
                    rates[cells[0]] = float(cells[5])
        if src != kernel_source_hash() or set(rates) != set(HIT_KERNELS):
            return None
        return rates
    except (OSError, ValueError, IndexError):
        return None


def cache_profile_run(torch, pti, dev, stream):
    """The kernels of the L2 hit-rate profile, a few launches each: the fused
    step, the SSQ GEMV alone, and the Q8 GEMV at N = 1, 2, 4 (17408x5120,
    weights rotated over copies)."""
    import synth
    L, sp = pti.lib(), pti._stream(stream)
    d = synth.twin(ROWS, COLS, synth.SEED_SSQ_FFN)
    P = pti.pack_ssq(d["A"], d["B"], d["sA"], d["sB"])
    n = copies_for(P.nbytes)
    w0 = torch.from_numpy(P).to(dev)
    ws = [w0] + [w0.clone() for _ in range(n - 1)]
    xa, xb = torch.from_numpy(d["xA"]).to(dev), torch.from_numpy(d["xB"]).to(dev)
    y2 = torch.empty((2, ROWS), dtype=torch.float32, device=dev)
    tok = torch.zeros(2, dtype=torch.int32, device=dev)
    am = torch.empty(2, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    work = pti.ssq_verify_workspace(dev)
    for i in range(12):
        pti._check("pti_gemv_ssq_verify", L.pti_gemv_ssq_verify(
            ws[i % n].data_ptr(), xa.data_ptr(), xb.data_ptr(), y2[0].data_ptr(), y2[1].data_ptr(), ROWS, COLS,
            tok.data_ptr(), am.data_ptr(), acc.data_ptr(), work.data_ptr(), work.numel(), sp))
        pti._check("pti_gemv_ssq", L.pti_gemv_ssq(ws[i % n].data_ptr(), xa.data_ptr(), xb.data_ptr(),
                                                  y2[0].data_ptr(), y2[1].data_ptr(), ROWS, COLS, sp))
    torch.cuda.synchronize()
    del ws, w0
    q = synth.q8(ROWS, COLS, 4, synth.SEED_Q8_FFN)
    Pq = pti.pack_q8(q["Q"], q["S"])
    nq = copies_for(Pq.nbytes)
    wq0 = torch.from_numpy(Pq).to(dev)
    wqs = [wq0] + [wq0.clone() for _ in range(nq - 1)]
    X = torch.from_numpy(q["X"]).to(dev)
    Y = torch.empty((4, ROWS), dtype=torch.float32, device=dev)
    for ns in (1, 2, 4):
        for i in range(12):
            pti._check("pti_gemv_q8_multi", L.pti_gemv_q8_multi(wqs[i % nq].data_ptr(), X.data_ptr(), Y.data_ptr(),
                                                                 ROWS, COLS, ns, sp))
    torch.cuda.synchronize()
    log("cache profile: 12 launches of each kernel")


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
        st = timed_stats(torch, lambda i: L.pti_verify_argmax(logits.data_ptr(), tok.data_ptr(), am.data_ptr(),
                                                              acc.data_ptr(), 32000, n, sp),
                         stream, reps=5, per_rep=50, warmup=10)
        out[f"verify_greedy_n{n}_v32000"] = st
        u = torch.rand(n, dtype=torch.float64, generator=g).to(dev)
        sw = pti.sample_verify_workspace(32000, n, dev)
        st = timed_stats(torch, lambda i: L.pti_sample_verify(logits.data_ptr(), tok.data_ptr(), u.data_ptr(), 0.7,
                                                              am.data_ptr(), acc.data_ptr(), 32000, n,
                                                              sw.data_ptr(), sw.numel(), sp),
                         stream, reps=5, per_rep=50, warmup=10)
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
        st = timed_stats(torch, lambda i: pti.attn_decode(q, kn, vn, kc[i % n_sets], vc[i % n_sets], pos, work,
                                                          out=o),
                         stream, reps=5, per_rep=50, warmup=10)
        kv_bytes = 2 * Hkv * d * 2 * ((L - 1) + L)  # K and V rows 0..pos of both streams
        algo = kv_bytes + 2 * S * H * d * 4 + 2 * S * Hkv * d * 4
        out[f"attn_twin_h40_kv8_d128_ctx{L}"] = {
            **st, "kv_bytes": kv_bytes, "algorithmic_bytes": algo, "cache_sets": n_sets,
            "GBps": round(algo / (st["median_us"] * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(algo / (st["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
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
                    help="time the fused SSQ step only, no other kernels (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 3 elementwise copies of 256 MiB (reference kernel for HBM byte counters)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from rocprofv3 CSV output (CPU only) and exit")
    ap.add_argument("--cache-profile", action="store_true",
                    help="run only the kernels of the L2 hit-rate profile (a few launches each) and exit")
    ap.add_argument("--summarize-hit-rate", metavar="TCC_DIR",
                    help="write the L2 hit-rate summary from rocprofv3 CSV output (CPU only) and exit")
    ap.add_argument("--profiles-out", default=os.path.join(HERE, "profiles"))
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles, args.profiles_out)
        return
    if args.summarize_hit_rate:
        summarize_hit_rate(args.summarize_hit_rate, args.profiles_out)
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
    if args.cache_profile:
        cache_profile_run(torch, pti, dev, stream)
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

    if args.copy_calibration:
        # torch.neg: an elementwise kernel that reads and writes 256 MiB each
        src = torch.ones(64 * 2**20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 x torch.neg over {src.numel() * 4} bytes")
        del src, dst
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
    per_kernel = {}
    copy_GBps = None
    if not args.only_main:
        st_gemv = timed_stats(torch, gemv, stream)
        st_verify = timed_stats(torch, verify, stream)
        ms_gemv = st_gemv["median_us"] * 1e-3
        log(f"unfused: ssq gemv alone {st_gemv}; verify alone {st_verify}")
        hr = read_hit_rates()
        per_kernel["ssq_twin_gemv_unfused"] = {**st_gemv,
                                               "weight_GBps": round(w_bytes / (ms_gemv * 1e-3) / 1e9, 2),
                                               "l2_hit_rate": hr["gemv_ssq_split_kernel<5, 2, false, 8>"] if hr else None}
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

    traffic = read_traffic()
    hit_rates = read_hit_rates()
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
            "traffic": traffic["bytes"] if traffic else None,
            "algorithmic_bytes_per_launch": algo_bytes,
            "avg_launch_us": round(ms_fused * 1e3, 3),
            "launch_us_stats": st_fused,
            "traffic_source": traffic["source"] if traffic else None,
            "vs_copy": round(algo_bytes / (ms_fused * 1e-3) / 1e9 / copy_GBps, 4) if copy_GBps else None,
            "rocprof_avg_us": read_kernel_avgs(),
            "rocprof_source": os.path.relpath(KT_FILE, HERE),
            "l2_hit_rate": ({k: hit_rates[k] for k in STEP_KERNELS} if hit_rates else None),
            "l2_hit_rate_source": os.path.relpath(HIT_FILE, HERE),
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
            per_kernel[f"q8_gemv_n{n}"] = {
                "us": round(t[n] * 1e3, 3), **stn,
                "weight_GBps": round(Pq.nbytes / (t[n] * 1e-3) / 1e9, 2),
                "frac_of_hbm_peak": round(algo / (t[n] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "gemv_per_s": round(1 / (t[n] * 1e-3), 1),
                "outputs_per_s": round(n * ROWS / (t[n] * 1e-3), 1),
                "l2_hit_rate": (hr or {}).get(Q8_KERNEL[n]),
            }
            log(f"q8 n={n}: {t[n] * 1e3:.2f} us, {Pq.nbytes / (t[n] * 1e-3) / 1e9:.1f} GB/s")
        per_kernel["q8_step_cost_n4_over_n1"] = round(t[4] / t[1], 4)
        del wqs, wq0
        torch.cuda.empty_cache()
        per_kernel.update(layer_and_graph(torch, pti, dev, stream))
        per_kernel.update(attention(torch, pti, dev, stream))
        per_kernel.update(verify_and_pack(torch, pti, dev, stream, d))
    result["per_kernel"] = per_kernel

    if not args.no_cpu:
        log("cpu baseline (oracle)...")
        result["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

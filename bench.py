"""Benchmark of the SP-region forward + backward on one MI355X.

A step is one pass of the whole region -- sp_region_fwd then sp_region_bwd --
over one token shard already resident in HBM.  The default workload is one
rank's shard of a 22B-class layer boundary (h=6144, s=2048, b=4, t=8:
[256, 4, 6144], bf16 I/O, LayerNorm, p=0.1).  Inputs are seeded synthetic
draws (sp_inputs.py).  Buffer sets are rotated so that consecutive steps miss
the 256 MB Infinity Cache.

Prints one JSON line: tokens/s, HBM GB/s and fraction of the 8 TB/s peak
from algorithmic bytes, the per-kernel times measured with HIP events on the
launch stream, the roofline record of the dominant kernel (with the HBM
traffic of the committed rocprofv3 counter summary, if it was taken on the
current kernel sources), and the CPU oracle timed on the host.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR    (writes profiles/..._hbm_traffic.json)
    python bench.py --stats-summary TRACE_DIR            (writes profiles/..._kernel_stats.md)
    python bench.py --counters-summary PMC_DIR [...]     (writes profiles/..._counters.md, one
                                                          directory per rocprofv3 --pmc pass)
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E
METRIC = "tokens/s and achieved HBM GB/s (% of peak) for SP-region fwd+bwd, 1 GPU"
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30             # the plain copy the counters are calibrated on


# The HIP sources each workload family runs: counter figures taken on other
# sources are stale.
REGION_SOURCES = ("sp_device.h", "sp_plan.h", "sp_host_checks.h", "sp_fwd.hip", "sp_bwd.hip",
                  "sp_region_api.hip")
ATTN_SOURCES = ("sp_device.h", "sp_plan.h", "sp_host_checks.h", "ring_attn.hip")


def kernel_source_hash(workload=None):
    from sp_inputs import ATTN_WORKLOADS
    names = ATTN_SOURCES if workload in ATTN_WORKLOADS else REGION_SOURCES
    h = hashlib.sha256()
    for n in names:
        h.update(n.encode())
        h.update(open(os.path.join(ROOT, "dropout_region_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def variant_bytes(w, variant):
    """Algorithmic bytes (fwd, bwd) of the two variants of the region.
    entry: fwd reads residual, writes y (+ stats); bwd reads dy, h (the
           residual) and the stats, writes dresidual, reads gamma, writes
           dgamma/dbeta.
    exit : fwd reads x, residual, writes h and the mask (+ bias); bwd reads
           dh_out and the mask, writes dx and dbias."""
    E, N, H = w.elems, w.rows, w.h
    es = 2 if w.io == 1 else 4
    ln = w.norm == 0
    n_stat = 2 if ln else 1
    if variant == "entry":
        fwd = E * 2 * es + (2 if ln else 1) * H * 4 + n_stat * N * 4
        bwd = E * 3 * es + n_stat * N * 4 + H * 4 + (2 if ln else 1) * H * 4
    else:
        m = 1 if w.p > 0 else 0
        fwd = E * (3 * es + m) + H * 4
        bwd = E * (2 * es + m) + H * 4
    return fwd, bwd


def algorithmic_bytes(w, with_bias=True, with_dh_out=False, mask_stored=True, x_parts=1):
    """Bytes the region must move per call (re-reads, partial sums and
    spills excluded).
    forward : read x (x_parts slabs of it with the reduce-scatter
              prologue), residual (es/elem each), write h, y (2 es/elem), mask
              (1 B/elem when p > 0), read bias/gamma/beta, write mean/rstd
    backward: read dy, h (2 es/elem), mask (1 B/elem), [dh_out] (es/elem),
              write dx, dres (2 es/elem), read gamma and the stats, write
              dgamma, dbeta, dbias
    Returns (fwd, bwd_rows, bwd_grads): bwd_rows is what the backward's row
    pass moves, bwd_grads the three gradient rows the finalize writes."""
    E, N, H = w.elems, w.rows, w.h
    es = 2 if w.io == 1 else 4
    m = 1 if w.p > 0 and mask_stored else 0
    ln = w.norm == 0
    n_par = (1 if with_bias else 0) + 1 + (1 if ln else 0)
    n_stat = 2 if ln else 1
    fwd = E * ((x_parts + 3) * es + m) + n_par * H * 4 + n_stat * N * 4
    n_grad = 1 + (1 if ln else 0) + 1
    bwd_rows = E * (4 * es + m + (es if with_dh_out else 0)) + n_stat * N * 4 + H * 4
    return fwd, bwd_rows, n_grad * H * 4


def _host_cpu():
    """(CPU model, logical CPUs the process may use, all logical CPUs)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return model, usable, os.cpu_count()


def cpu_baseline(w, seconds=6.0, max_threads=16):
    """The CPU oracle as it stands (plain C, one row at a time) on the same
    shard, forward + backward over all N rows, timed twice:
      - one thread, whole shard, repeated until `seconds` have passed;
      - every usable host core (at most max_threads: one GPU's share of the
        host), the rows cut into one contiguous range per thread, each thread
        running the oracle's forward then backward on its range (the oracle
        takes row ranges; ctypes releases the GIL during each call); the
        threads' parameter-gradient partials are added in thread order.
    Returns the all-core figure (tokens/s) with the one-thread one beside it."""
    import threading
    import numpy as np
    import oracle
    from oracle import build as obuild
    from sp_inputs import make_inputs
    if not os.path.exists(oracle.LIB_PATH):
        obuild.build_oracle()
    od = oracle.Desc(s_local=w.s_local, b=w.b, h=w.h, shard_index=0, t=w.t, io=w.io,
                     norm=w.norm, p=w.p, eps=w.eps, seed=w.seed, offset=0)
    inp = make_inputs(w.rows, w.h, w.io, seed=w.seed)
    beta = inp["beta"] if w.norm == 0 else None
    H = w.h

    def run_rows(r0, r1, out, slot):
        sl = slice(r0 * H, r1 * H)
        o = oracle.fwd(od, inp["x"][sl], inp["bias"], inp["residual"][sl], inp["gamma"], beta,
                       rows=(r0, r1))
        out[slot] = oracle.bwd(od, inp["dy"][sl], None, o["h"], o["mask"], o["mean"], o["rstd"],
                               inp["gamma"], rows=(r0, r1))

    def timed(fn):
        reps, total = 0, 0.0
        while total < seconds:
            t0 = time.perf_counter()
            fn()
            total += time.perf_counter() - t0
            reps += 1
        return reps, total

    one = [None]
    reps1, t1 = timed(lambda: run_rows(0, w.rows, one, 0))
    model, usable, nproc = _host_cpu()
    nt = max(1, min(usable, max_threads, w.rows))
    cuts = [w.rows * i // nt for i in range(nt + 1)]

    def all_cores():
        parts = [None] * nt
        th = [threading.Thread(target=run_rows, args=(cuts[i], cuts[i + 1], parts, i))
              for i in range(nt)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        grads = {k: np.zeros(H, np.float64) for k in ("dgamma", "dbeta", "dbias")}
        for p in parts:                       # thread order
            for k in grads:
                if p[k] is not None:
                    grads[k] += p[k]
        return grads

    repsn, tn = timed(all_cores)
    return {"value": round(w.rows * repsn / tn, 1), "unit": "tokens/s", "cores": nt,
            "kind": "oracle",
            "sample": f"whole shard [{w.s_local}, {w.b}, {w.h}] fwd+bwd x{repsn} on {nt} threads "
                      f"(rows cut into {nt} ranges; {tn:.1f} s); one thread: x{reps1} "
                      f"({t1:.1f} s)",
            "one_core": {"value": round(w.rows * reps1 / t1, 1), "cores": 1},
            "cpu_model": model, "nproc": nproc, "usable_cpus": usable}


def copy_bandwidth(torch, nbytes=COPY_BYTES, iters=20):
    """GB/s (read + write) of torch's device copy of a 1 GiB buffer (the HIP
    runtime's blit kernel): the plain copy the HBM counters are scaled by."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    sec = s.elapsed_time(e) / 1e3 / iters
    del src, dst
    return 2 * nbytes / sec / 1e9


# ------------------------------------------------------------------ summaries
def profile_key(workload, args):
    """Name of a workload's profile summaries: the workload, then the
    variant (entry, exit), the mask-free region (nomask), the reduce-scatter
    prologue (rsK) and any launch choice that is not the library's own."""
    key = workload
    if getattr(args, "variant", "full") != "full":
        key += "_" + args.variant
    if getattr(args, "no_mask", False):
        key += "_nomask"
    if getattr(args, "rs_parts", 0):
        key += f"_rs{args.rs_parts}"
    if getattr(args, "fwd_kernel", "auto") != "auto":
        key += f"_fwd{args.fwd_kernel}"
    if getattr(args, "bwd_path", "auto") != "auto":
        key += f"_bwd{args.bwd_path}"
    if getattr(args, "tile_rows", 0):
        key += f"_tile{args.tile_rows}"
    return key


def _profile_name(workload, what):
    prefix = "" if workload.startswith("ring_attn") else "sp_region_"
    return os.path.join(PROFILES, f"{prefix}{workload}_{what}")


def _short(name):
    """Readable kernel name: sp_region_fwd_kernel etc. (template arguments dropped)."""
    for base in ("sp_region_fwd_kernel", "sp_region_fwd_stream_kernel", "sp_region_bwd_rows_kernel",
                 "sp_region_bwd_rowsum_kernel", "sp_region_bwd_main_kernel",
                 "sp_region_bwd_finalize_kernel", "sp_region_bwd_exit_kernel",
                 "ring_attn_step_kernel", "ring_attn_merge_kernel"):
        if base in name:
            return base
    return name


def pmc_summary(fetch_dir, write_dir, workload, command):
    """Per-kernel HBM bytes per dispatch from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), scaled by what the same
    counter reads for the 1 GiB plain copy of the same run."""
    def load(d, counter):
        rows = list(csv.DictReader(open(glob.glob(os.path.join(d, "*counter_collection.csv"))[0])))
        by = {}
        for r in rows:
            if r["Counter_Name"] == counter:
                by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]) * 1024.0)
        return by
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy_name = [k for k in fetch if "copyBuffer" in k][0]
    f_scale = COPY_BYTES / max(fetch[copy_name])
    w_scale = COPY_BYTES / max(write[copy_name])
    out = {"command": command, "source_hash": kernel_source_hash(workload), "workload": workload,
           "copy_kernel": copy_name, "copy_bytes": COPY_BYTES,
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
    for k in fetch:
        if "sp_region" not in k and "ring_attn" not in k:
            continue
        wv = write.get(k, [0.0])
        out["kernels"][_short(k)] = {
            "fetch_bytes": round(sum(fetch[k]) / len(fetch[k]) * f_scale),
            "write_bytes": round(sum(wv) / len(wv) * w_scale), "dispatches": len(fetch[k])}
    path = _profile_name(workload, "hbm_traffic.json")
    json.dump(out, open(path, "w"), indent=1)
    print(path)


def stats_summary(trace_dir, workload, command):
    """Markdown table of a rocprofv3 --kernel-trace --stats run."""
    rows = list(csv.DictReader(open(glob.glob(os.path.join(trace_dir, "*kernel_stats.csv"))[0])))
    lines = [f"# rocprofv3 kernel statistics: {workload}", "",
             "Command (from the repository root, on the MI355X host):", "", "```", command, "```", "",
             f"Kernel sources: `{kernel_source_hash(workload)}` (hash of the workload's files in "
             "dropout_region_amd/csrc)", "",
             "| Kernel | Calls | Average ns | Min ns | Max ns | Share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                     f"{float(r['MinNs']):.0f} | {float(r['MaxNs']):.0f} | "
                     f"{float(r['Percentage']):.2f} |")
    path = _profile_name(workload, "kernel_stats.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


def counters_summary(pmc_dirs, workload, command):
    """Markdown table of the counters of one or more rocprofv3 --pmc runs (one
    per pass), averaged per dispatch for each kernel of the workload."""
    rows = []
    for pmc_dir in pmc_dirs:
        rows += list(csv.DictReader(open(glob.glob(os.path.join(pmc_dir, "*counter_collection.csv"))[0])))
    by = {}
    for r in rows:
        k = _short(r["Kernel_Name"])
        if not (k.startswith("sp_region") or k.startswith("ring_attn")):
            continue
        by.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 counters: {workload}", "", "Command (from the repository root, on the MI355X host):",
             "", "```", command, "```", "",
             f"Kernel sources: `{kernel_source_hash(workload)}` (hash of the workload's files in "
             "dropout_region_amd/csrc)", "", "Average per dispatch.", ""]
    for k, cs in by.items():
        lines += [f"## {k}", "", "| Counter | Value |", "|---|---|"]
        lines += [f"| {c} | {sum(v) / len(v):.6g} |" for c, v in sorted(cs.items())]
        lines.append("")
    path = _profile_name(workload, "counters.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


def load_traffic(workload):
    """Measured HBM bytes per dispatch by kernel, or None when no summary was
    taken on the current kernel sources."""
    path = _profile_name(workload, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    return t["kernels"] if t.get("source_hash") == kernel_source_hash(workload) else None


# ------------------------------------------------------------------ ring attention
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
ATTN_METRIC = "tokens/s and TFLOP/s (% of bf16 MFMA peak) for one rank's ring-attention forward, 1 GPU"


def attn_cpu_baseline(w, min_seconds=10.0):
    """The oracle (float64, one thread) on a bounded sample: query tokens
    [0, n) of the rank against every key of every block, all heads, doubled
    until it takes min_seconds.  Returns tokens/s scaled from the sample."""
    import oracle
    from oracle import build as obuild
    from sp_inputs import make_attn_inputs
    if not os.path.exists(oracle.LIB_PATH):
        obuild.build_oracle()
    od = oracle.AttnDesc(s_local=w.s_local, b=w.b, heads=w.heads, d=w.d, t=w.t)
    x = make_attn_inputs(w.s_local, w.b, w.heads, w.d, w.t, seed=w.seed)
    tok = w.b * w.heads * w.d
    n = 1
    while True:
        t0 = time.perf_counter()
        oracle.attention(od, x["q"][:n * tok], x["k"], x["v"], rows=(0, n))
        dt = time.perf_counter() - t0
        if dt >= min_seconds or n >= w.s_local:
            break
        n = min(w.s_local, n * 2 if dt < min_seconds / 4 else n + max(1, int(n * (min_seconds / dt - 1))))
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {w.s_local} query tokens x all {w.s} keys x {w.b * w.heads} "
                      f"(batch, head) pairs, float64 ({dt:.1f} s, 1 thread)"}


def bench_attention(args, w):
    import numpy as np
    import torch
    import dropout_region_amd as spr
    from sp_inputs import make_attn_inputs
    from tests import parity as P
    dev = torch.device("cuda:0")
    spr.lib()
    d = spr.AttnDesc(s_local=w.s_local, b=w.b, heads=w.heads, d=w.d, t=w.t, rank=0)
    print(f"[bench] ring attention {w.name}: {w.s_local} queries x {w.s} keys, {w.b}x{w.heads} "
          f"heads of {w.d} on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    x = make_attn_inputs(w.s_local, w.b, w.heads, w.d, w.t, seed=w.seed)
    q, k, v = (P.to_device(x[n], P.BF16) for n in ("q", "k", "v"))
    o = torch.empty(d.rows * d.d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(d.rows, dtype=torch.float32, device=dev)
    ws = torch.empty(spr.sp_ring_attn_workspace_bytes(d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        spr.sp_ring_attn_fwd(d, q, k, v, o, lse, ws, stream)

    if not args.no_parity:                       # sampled query tokens against the oracle
        import oracle
        from tests.attn_check import check_attention
        fwd()
        torch.cuda.synchronize()
        od = oracle.AttnDesc(s_local=w.s_local, b=w.b, heads=w.heads, d=w.d, t=w.t)
        tok, go, gl = w.b * w.heads * w.d, P.to_host(o), P.to_host(lse)
        for r in sorted({0, w.s_local // 2, w.s_local - 1}):
            qr = x["q"][r * tok:(r + 1) * tok]
            wo, wl = oracle.attention(od, qr, x["k"], x["v"], rows=(r, r + 1))
            check_attention(f"query {r}", od, qr, x["k"], x["v"], go[r * tok:(r + 1) * tok],
                            gl[r * w.b * w.heads:(r + 1) * w.b * w.heads], wo, wl,
                            rows=(r, r + 1))
        print("[bench] parity ok on sampled queries", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # Per-kernel times: the fused forward launched one index at a time (0: the
    # ring steps, 1: the merge of their partials), a HIP graph of 10 launches
    # of one index replayed between events on the launch stream.
    chunk = 10
    n_chunks = max(1, args.steps // chunk)
    cap_stream = torch.cuda.Stream()
    kernel_us = []
    for idx in range(spr.sp_ring_attn_fwd_num_launches(d)):
        g = torch.cuda.CUDAGraph()
        cap_stream.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap_stream):
            for _ in range(chunk):
                spr.sp_ring_attn_fwd_launch(d, idx, q, k, v, o, lse, ws, None)
        stream.wait_stream(cap_stream)
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(n_chunks):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        kernel_us.append(g0.elapsed_time(g1) / (n_chunks * chunk) * 1e3)
        del g
    step_us, merge_us = kernel_us
    tflops = w.flops / (step_us * 1e-6) / 1e12
    out = {
        "metric": ATTN_METRIC, "value": round(w.s_local / (ms / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "s": w.s, "t": w.t, "rank": 0, "queries": w.s_local,
                   "b": w.b, "heads": w.heads, "head_dim": w.d, "causal": False},
        "tflops": round(w.flops / (ms * 1e-3) / 1e12, 1),
        "kernels_us": {"ring_attn_step_kernel": round(step_us, 2),
                       "ring_attn_merge_kernel": round(merge_us, 2)},
        "kernel_timing": "HIP events around replays of a HIP graph of 10 launches of one kernel",
        "roofline": {"bound": "mfma", "kernel": "ring_attn_step_kernel", "achieved": round(tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "algorithmic_flops_per_launch": w.flops, "launch_us": round(step_us, 2)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = attn_cpu_baseline(w)
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ bench
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--min-set-bytes", type=float, default=1.0, help="GiB of rotated buffers")
    ap.add_argument("--rs-parts", type=int, default=0,
                    help="forward with the reduce-scatter prologue over this many partial "
                         "slabs (sp_region_fwd_rs); 0 = the plain forward")
    ap.add_argument("--variant", choices=("full", "entry", "exit"), default="full",
                    help="entry: the norm-only entry (no x, p = 0); exit: the norm-free exit "
                         "(no norm; backward sp_region_bwd_exit)")
    ap.add_argument("--no-mask", action="store_true",
                    help="mask-free region: the forward stores no mask, the backward "
                         "regenerates the dropout decisions")
    ap.add_argument("--fwd-kernel", choices=("auto", "rows", "stream"), default="auto",
                    help="the forward kernel (a launch choice of the descriptor)")
    ap.add_argument("--bwd-path", choices=("auto", "fused", "split"), default="auto",
                    help="the backward path (a launch choice of the descriptor)")
    ap.add_argument("--tile-rows", type=int, default=0,
                    help="rows per tile of the split backward and the exit (0: the library's)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--stats-summary", metavar="TRACE_DIR")
    ap.add_argument("--counters-summary", nargs="+", metavar="PMC_DIR")
    ap.add_argument("--command", default="", help="command recorded in a summary")
    args = ap.parse_args()

    from sp_inputs import HEADLINE, WORKLOADS
    wname = args.workload or HEADLINE
    key = profile_key(wname, args)
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary, key, args.command)
    if args.stats_summary:
        return stats_summary(args.stats_summary, key, args.command)
    if args.counters_summary:
        return counters_summary(args.counters_summary, key, args.command)
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(the region is per-rank; there are no collectives to run)", file=sys.stderr)
        sys.exit(2)

    from sp_inputs import ATTN_WORKLOADS
    if wname in ATTN_WORKLOADS:
        return bench_attention(args, ATTN_WORKLOADS[wname])

    import numpy as np
    import torch
    import dropout_region_amd as spr
    from sp_inputs import make_inputs
    from tests import parity as P

    w = WORKLOADS[wname]
    dev = torch.device("cuda:0")
    V = args.variant
    d = spr.Desc(s_local=w.s_local, b=w.b, h=w.h, shard_index=0, t=w.t, io=w.io, norm=w.norm,
                 p=0.0 if V == "entry" else w.p, eps=w.eps, seed=w.seed, offset=0,
                 fwd_kernel={"auto": 0, "rows": 1, "stream": 2}[args.fwd_kernel],
                 bwd_path={"auto": 0, "fused": 1, "split": 2}[args.bwd_path],
                 bwd_tile_rows=args.tile_rows)
    if V != "full" and (args.rs_parts or args.no_mask):
        sys.exit("bench.py: --variant takes neither --rs-parts nor --no-mask")
    spr.lib()
    print(f"[bench] workload {w.name}: shard [{w.s_local}, {w.b}, {w.h}] N={w.rows} "
          f"on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    inp = make_inputs(w.rows, w.h, w.io, seed=w.seed)
    K = args.rs_parts
    parts_host = None
    if K:
        from sp_inputs import make_parts
        parts_host = make_parts(w.rows, w.h, w.io, K, seed=w.seed)

    # ---- parity first: sampled rows against the oracle
    if not args.no_parity:
        import oracle
        od = oracle.Desc(**{k: getattr(d, k) for k in ("s_local", "b", "h", "shard_index", "t",
                                                         "io", "norm", "p", "eps", "seed",
                                                         "offset")})
        if V != "full":
            ln = w.norm == 0
            rr = slice(0, 2 * w.h)
            odv = oracle.Desc(**{**od.__dict__, "s_local": 2, "b": 1})    # rows 0 and 1
            dv = spr.Desc(**{**d.__dict__, "s_local": 2, "b": 1})
            sub = {k: (v[rr] if k in ("x", "residual") else v) for k, v in inp.items()}
            dev_in = {k: P.to_device(sub[k], w.io) for k in ("x", "residual")}
            if V == "entry":
                want = oracle.fwd(odv, None, None, sub["residual"], sub["gamma"],
                                  sub["beta"] if ln else None)
                g = spr.fwd(dv, None, None, dev_in["residual"], P.to_device(sub["gamma"]),
                            P.to_device(sub["beta"]) if ln else None, write_h=False)
                P.io_close("y", P.to_host(g["y"]), want["y"], w.io)
            else:
                want = oracle.fwd(odv, sub["x"], sub["bias"], sub["residual"], None, None)
                g = spr.fwd(dv, dev_in["x"], P.to_device(sub["bias"]), dev_in["residual"],
                            None, None)
                P.exact("h", P.to_host(g["h"]), want["h"])
                if want["mask"] is not None:
                    P.exact("mask", P.to_host(g["mask"]), want["mask"])
            print(f"[bench] {V} parity ok on rows [0, 1]", file=sys.stderr, flush=True)
        elif K:
            ref_inp = dict(inp, x=oracle.reduce_parts(od, parts_host))
            got = P.gpu_fwd_rs(d, inp, parts_host, K)
        else:
            ref_inp = inp
            got = P.gpu_fwd(d, inp, store_mask=not args.no_mask)
        if V == "full":
            rows = sorted({0, 1, w.rows // 2, w.rows - 1})
            for r in rows:
                sl, st = slice(r * w.h, (r + 1) * w.h), slice(r, r + 1)
                want = P.oracle_fwd(od, ref_inp, rows=(r, r + 1))
                if args.no_mask:
                    want["mask"] = None
                P.check_fwd({k: (v[sl] if k in ("h", "y", "mask") else v[st])
                             if v is not None else None for k, v in got.items()}, want, w.io)
            print(f"[bench] parity ok on rows {rows}", file=sys.stderr, flush=True)

    # ---- device buffers: rotate sets so consecutive steps miss the MALL
    es = 2 if w.io == 1 else 4
    x0 = P.to_device(inp["x"], w.io)
    parts0 = P.to_device(parts_host.ravel(), w.io) if K else None
    r0 = P.to_device(inp["residual"], w.io)
    dy0 = P.to_device(inp["dy"], w.io)
    bias, gamma = P.to_device(inp["bias"]), P.to_device(inp["gamma"])
    beta = P.to_device(inp["beta"]) if w.norm == 0 else None
    set_bytes = w.elems * ((7 + K) * es + 1)
    nsets = max(2, int(np.ceil(args.min_set_bytes * (1 << 30) / set_bytes)))
    sets = []
    for _ in range(nsets):
        s = {"x": x0.clone(), "res": r0.clone(), "dy": dy0.clone()}
        if K:
            s["parts"] = parts0.clone()
        s.update(spr.alloc_fwd_outputs(d, dev, store_mask=not args.no_mask))
        s.update({("b_" + k): v for k, v in spr.alloc_bwd_outputs(d, dev).items()})
        sets.append(s)
    stream = torch.cuda.current_stream()
    n_bwd = spr.sp_region_bwd_num_launches(d)

    def fwd(s, stream=stream):
        if V == "entry":
            spr.sp_region_fwd(d, None, None, s["res"], gamma, beta, None, s["y"], None,
                              s["mean"], s["rstd"], stream)
        elif V == "exit":
            spr.sp_region_fwd(d, s["x"], bias, s["res"], None, None, s["h"], None, s["mask"],
                              None, None, stream)
        elif K:
            spr.sp_region_fwd_rs(d, s["parts"], K, bias, s["res"], gamma, beta, s["h"], s["y"],
                                 s["mask"], s["mean"], s["rstd"], stream)
        else:
            spr.sp_region_fwd(d, s["x"], bias, s["res"], gamma, beta, s["h"], s["y"], s["mask"],
                              s["mean"], s["rstd"], stream)

    def bwd_args(s):
        if V == "entry":            # h is the residual; no x, so no dx and no dbias
            return (s["dy"], None, s["res"], None, s["mean"], s["rstd"], gamma, None,
                    s["b_dres"], s["b_dgamma"], s["b_dbeta"], None, s["b_workspace"])
        return (s["dy"], None, s["h"], s["mask"], s["mean"], s["rstd"], gamma, s["b_dx"],
                s["b_dres"], s["b_dgamma"], s["b_dbeta"], s["b_dbias"], s["b_workspace"])

    def bwd(s, stream=stream):
        if V == "exit":             # dh_out drawn as dy
            spr.sp_region_bwd_exit(d, s["dy"], s["mask"], s["b_dx"], s["b_dbias"],
                                   s["b_workspace"], stream)
        else:
            spr.sp_region_bwd(d, *bwd_args(s), stream)

    if V == "exit":
        n_bwd = 1                   # sp_region_bwd_exit: exit kernel + finalize

    for i in range(args.warmup):
        fwd(sets[i % nsets])
        bwd(sets[i % nsets])
    torch.cuda.synchronize()

    # ---- timed region 1: whole steps, nothing between the calls
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        s = sets[i % nsets]
        fwd(s)
        bwd(s)
    t_enqueued = time.perf_counter() - t0
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # ---- the same steps with an event after every `per` steps: the
    # distribution (median, p10, p90) of the step time averaged over each
    # group of `per` (an event after every step would itself add ~2 us a step)
    per = 5

    def step_times(order):
        n = max(1, args.steps // per)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for c in range(n):
            for i in range(c * per, (c + 1) * per):
                order(i)
            evs[c + 1].record(stream)
        torch.cuda.synchronize()
        return np.array([evs[c].elapsed_time(evs[c + 1]) / per for c in range(n)]) * 1e3

    def same_set(i):
        s = sets[i % nsets]
        fwd(s)
        bwd(s)

    # The backward of step i reads the set the forward of step i - nsets/2
    # wrote: h and the mask were written half the rotation (>= 512 MB of
    # traffic) earlier, so they come from HBM, not from the Infinity Cache a
    # same-set step may find them in.
    lag = nsets // 2

    def lagged(i):
        fwd(sets[i % nsets])
        bwd(sets[(i - lag) % nsets])

    per_step_us = step_times(same_set)
    lagged_us = step_times(lagged)

    # ---- timed region 2: each kernel alone.  A chunk of back-to-back
    # launches of one kernel is captured in a HIP graph and replayed between
    # two HIP events on the stream, so the host's launch rate does not show
    # in a short kernel's time.  Kernel k runs over the buffer sets after
    # kernel k-1 has run over all of them, so every launch reads what the
    # launch before it in the sequence wrote for the same set (the backward
    # launched one index at a time: the launches sp_region_bwd makes).
    nk = 1 + n_bwd
    chunk = 10
    n_chunks = max(1, args.steps // chunk)
    per_kernel_ms = np.zeros((n_chunks, nk))
    cap_stream = torch.cuda.Stream()
    for k in range(nk):
        def launches():
            for i in range(chunk):
                s = sets[i % nsets]
                if k == 0:
                    fwd(s, stream=None)          # the capture stream
                elif V == "exit":
                    bwd(s, stream=None)
                else:
                    spr.sp_region_bwd_launch(d, k - 1, *bwd_args(s))
        g = torch.cuda.CUDAGraph()
        cap_stream.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap_stream):
            launches()
        stream.wait_stream(cap_stream)
        g.replay()
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_chunks + 1)]
        evs[0].record(stream)
        for c in range(n_chunks):
            g.replay()
            evs[c + 1].record(stream)
        torch.cuda.synchronize()
        per_kernel_ms[:, k] = [evs[c].elapsed_time(evs[c + 1]) / chunk for c in range(n_chunks)]
        del g
    kernel_us = per_kernel_ms.mean(axis=0) * 1e3

    # ---- whole steps (fwd then bwd) captured as a HIP graph of `chunk` steps
    # and replayed: the GPU's step time without the host's launch path (a
    # diagnostic; `value` is the eager step above)
    g = torch.cuda.CUDAGraph()
    cap_stream.wait_stream(stream)
    with torch.cuda.graph(g, stream=cap_stream):
        for i in range(chunk):
            fwd(sets[i % nsets], stream=None)
            bwd(sets[i % nsets], stream=None)
    stream.wait_stream(cap_stream)
    g.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(n_chunks):
        g.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_step_us = g0.elapsed_time(g1) / (n_chunks * chunk) * 1e3
    del g

    # ---- whole steps as above, with the backward's last launch (the
    # fixed-order column finalize of dgamma/dbeta/dbias) on a second stream
    # so that it overlaps the next step's forward, as a training step may
    # schedule it (nothing downstream of the region's backward reads the
    # parameter gradients before the optimizer).  Forked from and joined to
    # the capture stream inside the graph; every launch is replayed.
    graph_overlap_us = None
    if V == "full" and n_bwd >= 2 and chunk <= nsets:
        side = torch.cuda.Stream()               # default priority
        g = torch.cuda.CUDAGraph()
        cap_stream.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap_stream):
            for i in range(chunk):               # distinct sets: no reuse inside the graph
                s = sets[i % nsets]
                fwd(s, stream=None)
                for k in range(n_bwd - 1):
                    spr.sp_region_bwd_launch(d, k, *bwd_args(s), None)
                side.wait_stream(cap_stream)
                spr.sp_region_bwd_launch(d, n_bwd - 1, *bwd_args(s), side)
            cap_stream.wait_stream(side)
        stream.wait_stream(cap_stream)
        g.replay()
        torch.cuda.synchronize()
        g0.record(stream)
        for _ in range(n_chunks):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_overlap_us = g0.elapsed_time(g1) / (n_chunks * chunk) * 1e3
        del g

    # ---- the reduce-scatter prologue against its unfused form (torch's sum of
    # the slabs, fp32 accumulation, into x; then sp_region_fwd), eager
    rs = None
    if K:
        xs = torch.empty(w.elems, dtype=x0.dtype, device=dev)

        def unfused(s, with_fwd=True):
            torch.sum(s["parts"].view(K, -1), dim=0, out=xs)
            if with_fwd:
                spr.sp_region_fwd(d, xs, bias, s["res"], gamma, beta, s["h"], s["y"], s["mask"],
                                  s["mean"], s["rstd"], stream)

        def eager_us(fn):
            for i in range(3):
                fn(sets[i % nsets])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.steps):
                fn(sets[i % nsets])
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps * 1e3

        rs = {"nparts": K, "fused_fwd_us": round(float(kernel_us[0]), 2),
              "unfused_sum_plus_fwd_us": round(eager_us(unfused), 2),
              "unfused_sum_us": round(eager_us(lambda s: unfused(s, False)), 2),
              "fused_fwd_eager_us": round(eager_us(fwd), 2)}

    # ---- layers of two calls (pre-attention and pre-MLP): call B's residual
    # is call A's h, and call A's backward takes call B's dresidual as dh_out
    layer = None
    if w.calls_per_layer == 2 and V == "full":
        def layer_step(sA, sB):
            spr.sp_region_fwd(dA, sA["x"], bias, sA["res"], gamma, beta, sA["h"], sA["y"],
                              sA["mask"], sA["mean"], sA["rstd"], stream)
            spr.sp_region_fwd(dB, sB["x"], bias, sA["h"], gamma, beta, sB["h"], sB["y"],
                              sB["mask"], sB["mean"], sB["rstd"], stream)
            spr.sp_region_bwd(dB, *bwd_args(sB), stream)
            spr.sp_region_bwd(dA, sA["dy"], sB["b_dres"], *bwd_args(sA)[2:], stream)
        dA = d
        dB = spr.Desc(**{**d.__dict__, "offset": 1})
        pairs = [(sets[i], sets[(i + 1) % nsets]) for i in range(0, nsets, 2)]
        for i in range(2):
            layer_step(*pairs[i % len(pairs)])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            layer_step(*pairs[i % len(pairs)])
        e1.record(stream)
        torch.cuda.synchronize()
        layer_ms = e0.elapsed_time(e1) / args.steps
        fA, rA, gA = algorithmic_bytes(w, with_dh_out=True, mask_stored=not args.no_mask)
        fB, rB, gB = algorithmic_bytes(w, mask_stored=not args.no_mask)
        layer_bytes = fA + rA + gA + fB + rB + gB
        layer = {"calls": 2, "ms_per_layer": round(layer_ms, 5),
                 "tokens_per_s": round(w.rows / (layer_ms / 1e3), 1),
                 "hbm_gbps": round(layer_bytes / (layer_ms / 1e3) / 1e9, 1),
                 "algorithmic_bytes": layer_bytes}

    # launch 0 is sp_region_fwd: its row kernel or its stream kernel
    names = ["sp_region_fwd"] + (["sp_region_bwd_exit"] if V == "exit" else
        ["sp_region_bwd_rows_kernel", "sp_region_bwd_finalize_kernel"] if n_bwd == 2 else
        ["sp_region_bwd_rowsum_kernel", "sp_region_bwd_main_kernel", "sp_region_bwd_finalize_kernel"])
    fwd_b, bwd_rows_b, bwd_grad_b = algorithmic_bytes(w, mask_stored=not args.no_mask,
                                                      x_parts=max(K, 1))
    if V != "full":
        fwd_b, bwd_rows_b = variant_bytes(w, V)
        bwd_grad_b = 0
    # algorithmic bytes of each launch (the split path's row-sum pass only re-reads)
    alg = [fwd_b] + ([bwd_rows_b] if V == "exit" else
                     [bwd_rows_b, bwd_grad_b] if n_bwd == 2 else [0, bwd_rows_b, bwd_grad_b])

    tokens_per_s = w.rows / (ms_per_step / 1e3)
    total_alg = fwd_b + bwd_rows_b + bwd_grad_b
    gbps = total_alg / (ms_per_step / 1e3) / 1e9
    dom = int(np.argmax(kernel_us))
    achieved = alg[dom] / (kernel_us[dom] / 1e6) / 1e9
    traffic = load_traffic(profile_key(w.name, args))
    dom_traffic = None
    aliases = {"sp_region_fwd": ("sp_region_fwd_kernel", "sp_region_fwd_stream_kernel")}
    for kname in aliases.get(names[dom], (names[dom],)):
        if traffic and kname in traffic:
            t = traffic[kname]
            dom_traffic = t["fetch_bytes"] + t["write_bytes"]
    copy_gbps = copy_bandwidth(torch)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.io == 1 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "shard": [w.s_local, w.b, w.h], "t": w.t,
                   "norm": "layernorm" if w.norm == 0 else "rmsnorm", "p": w.p, "eps": w.eps,
                   "io": "bf16" if w.io == 1 else "fp32", "params_and_stats": "fp32",
                   "tokens_per_step": w.rows, "buffer_sets": nsets,
                   "mask": ("regenerated in the backward" if args.no_mask else "stored uint8")
                   if w.p > 0 else "none (p = 0)"},
        "hbm_gbps": round(gbps, 1), "hbm_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "copy_gbps": round(copy_gbps, 1), "frac_of_copy": round(gbps / copy_gbps, 4),
        "launch_choices": {"fwd_kernel": args.fwd_kernel, "bwd_path": args.bwd_path,
                           "bwd_tile_rows": args.tile_rows or "auto"},
        "kernels_us": {n: round(float(u), 2) for n, u in zip(names, kernel_us)},
        "kernels_us_p10_p90": {n: [round(float(np.percentile(per_kernel_ms[:, k], q)) * 1e3, 2)
                                   for q in (10, 90)] for k, n in enumerate(names)},
        "kernel_timing": f"HIP events around replays of a HIP graph of {chunk} launches of one kernel",
        "algorithmic_bytes": {"fwd": fwd_b, "bwd": bwd_rows_b + bwd_grad_b},
        "step_us_median": round(float(np.median(per_step_us)), 2),
        "step_us_p10_p90": [round(float(np.percentile(per_step_us, q)), 2) for q in (10, 90)],
        "step_us_lagged_bwd_median": round(float(np.median(lagged_us)), 2),
        "graph_step_us_finalize_on_second_stream": (round(graph_overlap_us, 2)
                                                    if graph_overlap_us is not None else None),
        "step_timing": "ms_per_step and value: HIP events around all K steps; step_us_*: an event "
                       f"after every {per} steps (a second pass of K steps), the distribution of "
                       "those groups' mean step; lagged_bwd: the backward "
                       f"of step i reads the set step i - {lag} wrote; graph_step_us: whole steps "
                       "replayed from a HIP graph; ..._finalize_on_second_stream: the same with "
                       "the backward's column finalize on a second stream, overlapping the next "
                       "forward",
        "wall_s_timed_region": round(wall, 4),
        "host_enqueue_us_per_step": round(t_enqueued / args.steps * 1e6, 2),
        "graph_step_us": round(graph_step_us, 2),
        "roofline": {"bound": "hbm", "kernel": names[dom], "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": dom_traffic, "algorithmic_bytes_per_launch": alg[dom],
                     "launch_us": round(float(kernel_us[dom]), 2)},
    }
    if layer is not None:
        out["layer"] = layer
    if rs is not None:
        out["rs_prologue"] = rs
        out["config"]["rs_parts"] = K
    if V != "full":
        out["config"]["variant"] = {"entry": "norm-only entry (no x, p = 0)",
                                    "exit": "norm-free exit (no norm)"}[V]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

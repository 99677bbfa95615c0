"""Benchmark of the SP-region forward + backward on one MI355X.

A step is one pass of the whole region -- sp_region_fwd then sp_region_bwd --
over one token shard that is already resident in HBM.  The default workload
is one rank's shard of a 22B-class layer boundary (h=6144, s=2048, b=4,
t=8: [256, 4, 6144], bf16 I/O, LayerNorm, p=0.1).  Inputs are seeded
synthetic draws (sp_inputs.py).  Buffer sets are rotated so that the working
set of consecutive steps exceeds the 256 MB Infinity Cache.

Prints one JSON line: tokens/s, HBM GB/s and fraction of the 8 TB/s peak
from algorithmic bytes, per-call times measured with HIP events on the
launch stream, the roofline record of the dominant kernel, and the CPU
oracle timed on the host (a baseline, not a target).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0           # MI355X HBM3E
METRIC = "tokens/s and achieved HBM GB/s (% of peak) for SP-region fwd+bwd, 1 GPU"


def algorithmic_bytes(w, with_bias=True, with_dh_out=False):
    """Bytes the region must move per call (re-reads, partial sums and
    spills excluded).
    forward : read x, residual (2 es/elem), write h, y (2 es/elem), mask
              (1 B/elem when p > 0), read bias/gamma/beta, write mean/rstd
    backward: read dy, h (2 es/elem), mask (1 B/elem), [dh_out] (es/elem),
              write dx, dres (2 es/elem), read gamma and the stats, write
              dgamma, dbeta, dbias"""
    E, N, H = w.elems, w.rows, w.h
    es = 2 if w.io == 1 else 4
    m = 1 if w.p > 0 else 0
    ln = w.norm == 0
    n_par = (1 if with_bias else 0) + 1 + (1 if ln else 0)
    n_stat = 2 if ln else 1
    fwd = E * (4 * es + m) + n_par * H * 4 + n_stat * N * 4
    n_grad = 1 + (1 if ln else 0) + 1
    bwd = E * (4 * es + m + (es if with_dh_out else 0)) + n_stat * N * 4 + H * 4 + n_grad * H * 4
    return fwd, bwd


def cpu_baseline(w, min_seconds=10.0, max_seconds=30.0):
    """The CPU oracle (single-threaded C, as it stands) on the same shard:
    forward + backward over all N rows, repeated until at least min_seconds
    of CPU time have passed.  Returns tokens/s and the sample description."""
    import oracle
    from oracle import build as obuild
    from sp_inputs import make_inputs
    if not os.path.exists(oracle.LIB_PATH):
        obuild.build_oracle()
    od = oracle.Desc(s_local=w.s_local, b=w.b, h=w.h, shard_index=0, t=w.t, io=w.io,
                     norm=w.norm, p=w.p, eps=w.eps, seed=w.seed, offset=0)
    inp = make_inputs(w.rows, w.h, w.io, seed=w.seed)
    beta = inp["beta"] if w.norm == 0 else None
    reps, t_total = 0, 0.0
    while t_total < min_seconds and t_total < max_seconds:
        t0 = time.perf_counter()
        o = oracle.fwd(od, inp["x"], inp["bias"], inp["residual"], inp["gamma"], beta)
        oracle.bwd(od, inp["dy"], None, o["h"], o["mask"], o["mean"], o["rstd"], inp["gamma"])
        t_total += time.perf_counter() - t0
        reps += 1
    return {"value": w.rows * reps / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"whole shard [{w.s_local}, {w.b}, {w.h}] fwd+bwd x{reps} "
                      f"({t_total:.1f} s, 1 thread)"}


def copy_bandwidth(torch, nbytes=1 << 30, iters=20):
    """GB/s (read + write) of torch's device copy of a 1 GiB buffer."""
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--min-set-bytes", type=float, default=1.0, help="GiB of rotated buffers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the region is per-rank; there are no collectives to run)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import dropout_region_amd as spr
    from sp_inputs import HEADLINE, WORKLOADS, make_inputs
    from tests import parity as P

    w = WORKLOADS[args.workload or HEADLINE]
    dev = torch.device("cuda:0")
    d = spr.Desc(s_local=w.s_local, b=w.b, h=w.h, shard_index=0, t=w.t, io=w.io, norm=w.norm,
                 p=w.p, eps=w.eps, seed=w.seed, offset=0)
    spr.lib()
    print(f"[bench] workload {w.name}: shard [{w.s_local}, {w.b}, {w.h}] N={w.rows} "
          f"on {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    inp = make_inputs(w.rows, w.h, w.io, seed=w.seed)

    # ---- parity first: sampled rows against the oracle
    if not args.no_parity:
        import oracle
        od = oracle.Desc(**{k: getattr(d, k) for k in ("s_local", "b", "h", "shard_index", "t",
                                                         "io", "norm", "p", "eps", "seed",
                                                         "offset")})
        got = P.gpu_fwd(d, inp)
        rows = sorted({0, 1, w.rows // 2, w.rows - 1})
        for r in rows:
            sl, st = slice(r * w.h, (r + 1) * w.h), slice(r, r + 1)
            want = P.oracle_fwd(od, inp, rows=(r, r + 1))
            P.check_fwd({k: (v[sl] if k in ("h", "y", "mask") else v[st]) if v is not None else None
                         for k, v in got.items()}, want, w.io)
        print(f"[bench] parity ok on rows {rows}", file=sys.stderr, flush=True)

    # ---- device buffers: rotate sets so consecutive steps miss the MALL
    es = 2 if w.io == 1 else 4
    x0 = P.to_device(inp["x"], w.io)
    r0 = P.to_device(inp["residual"], w.io)
    dy0 = P.to_device(inp["dy"], w.io)
    bias, gamma = P.to_device(inp["bias"]), P.to_device(inp["gamma"])
    beta = P.to_device(inp["beta"]) if w.norm == 0 else None
    set_bytes = w.elems * (7 * es + 1)
    nsets = max(2, int(np.ceil(args.min_set_bytes * (1 << 30) / set_bytes)))
    sets = []
    for _ in range(nsets):
        s = {"x": x0.clone(), "res": r0.clone(), "dy": dy0.clone()}
        s.update(spr.alloc_fwd_outputs(d, dev))
        s.update({("b_" + k): v for k, v in spr.alloc_bwd_outputs(d, dev).items()})
        sets.append(s)
    stream = torch.cuda.current_stream()

    def fwd(s):
        spr.sp_region_fwd(d, s["x"], bias, s["res"], gamma, beta, s["h"], s["y"], s["mask"],
                          s["mean"], s["rstd"], stream)

    def bwd(s):
        spr.sp_region_bwd(d, s["dy"], None, s["h"], s["mask"], s["mean"], s["rstd"], gamma,
                          s["b_dx"], s["b_dres"], s["b_dgamma"], s["b_dbeta"], s["b_dbias"],
                          s["b_workspace"], stream)

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
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # ---- timed region 2: HIP events around each call on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        s = sets[i % nsets]
        evs[i][0].record(stream)
        fwd(s)
        evs[i][1].record(stream)
        bwd(s)
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    fwd_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    bwd_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    fwd_b, bwd_b = algorithmic_bytes(w)
    tokens_per_s = w.rows / (ms_per_step / 1e3)
    gbps = (fwd_b + bwd_b) / (ms_per_step / 1e3) / 1e9
    f_us, b_us = float(np.mean(fwd_ms) * 1e3), float(np.mean(bwd_ms) * 1e3)
    dom, dom_b, dom_us = ("sp_region_bwd", bwd_b, b_us) if b_us >= f_us else ("sp_region_fwd", fwd_b, f_us)
    achieved = dom_b / (dom_us / 1e6) / 1e9
    copy_gbps = copy_bandwidth(torch)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if w.io == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "shard": [w.s_local, w.b, w.h], "t": w.t,
                   "norm": "layernorm" if w.norm == 0 else "rmsnorm", "p": w.p, "eps": w.eps,
                   "io": "bf16" if w.io == 1 else "fp32", "params_and_stats": "fp32",
                   "tokens_per_step": w.rows, "buffer_sets": nsets},
        "hbm_gbps": round(gbps, 1), "hbm_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
        "copy_gbps": round(copy_gbps, 1), "frac_of_copy": round(gbps / copy_gbps, 4),
        "fwd_us": round(f_us, 2), "bwd_us": round(b_us, 2),
        "fwd_us_p10_p90": [round(float(np.percentile(fwd_ms, q)) * 1e3, 2) for q in (10, 90)],
        "bwd_us_p10_p90": [round(float(np.percentile(bwd_ms, q)) * 1e3, 2) for q in (10, 90)],
        "algorithmic_bytes": {"fwd": fwd_b, "bwd": bwd_b},
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

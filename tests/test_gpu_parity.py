"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Masks and h must be bit-exact; y, the statistics and the gradients must meet
the tolerances in tests/parity.py.  Every backward check feeds both sides the
oracle's saved tensors (so the backward is checked alone), runs the GPU call
twice into the same buffers (results must be bit-identical), and also runs
the GPU backward from the GPU forward's own saved tensors (the chain).
"""
import zlib

import numpy as np
import pytest

import dropout_region_amd as spr
import oracle
from sp_inputs import WORKLOADS, make_inputs, make_parts
from tests import parity as P

pytestmark = pytest.mark.gpu

F32, BF16, LN, RMS = spr.SPR_F32, spr.SPR_BF16, spr.SPR_LAYERNORM, spr.SPR_RMSNORM


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    spr.lib()                            # raises if the HIP library is missing


def descs(**kw):
    return spr.Desc(**kw), oracle.Desc(**kw)


def run_case(name, kw, seed=0, with_bias=True, with_dh_out=False, want_dbias=True,
             paths=(None,), fwd_paths=(None,), tile_rows=None):
    """paths: backward paths to check (None = the library's own choice,
    "fused", "split"); fwd_paths: forward kernels (None, "rows", "stream");
    tile_rows: rows per tile of the split backward (None: the library's)."""
    d, od = descs(**kw)
    d = P.tuned(d, tile_rows=tile_rows)
    _say(f"[case] {name}: {kw} bias={with_bias} dh_out={with_dh_out} dbias={want_dbias}")
    inp = make_inputs(d.rows, d.h, d.io, seed=seed, dh_out=with_dh_out)
    want = P.oracle_fwd(od, inp, with_bias)
    for fpath in fwd_paths:
        _say(f"[case] {name}: forward kernel {fpath or 'auto'}")
        got = P.gpu_fwd(d, inp, with_bias, path=fpath)
        P.check_fwd(got, want, d.io)
    wb = P.oracle_bwd(od, inp, want, with_dh_out, want_dbias)
    for path in paths:
        _say(f"[case] {name}: backward path {path or 'auto'}")
        gb = P.gpu_bwd(d, inp, want, with_dh_out, want_dbias, repeat=2, path=path)
        P.check_bwd(gb, wb, d.io)
        gc = P.gpu_bwd(d, inp, got, with_dh_out, want_dbias, path=path)
        P.check_bwd(gc, wb, d.io)
    return inp, got, gb


def base(**kw):
    b = dict(s_local=8, b=2, h=256, shard_index=0, t=1, io=BF16, norm=LN, p=0.1, eps=1e-5,
             seed=0, offset=0)
    b.update(kw)
    return b


SMALL = {
    "fp32_ln_h256_shard1of2": base(s_local=64, h=256, shard_index=1, t=2, io=F32),
    "bf16_ln_h6144_shard5of8": base(s_local=10, b=3, h=6144, shard_index=5, t=8),
    "bf16_rms_h8192_p0": base(s_local=17, b=1, h=8192, norm=RMS, p=0.0, eps=1e-6),
    "bf16_rms_h8192_p0.1": base(s_local=17, b=1, h=8192, norm=RMS, p=0.1, eps=1e-6),
    "bf16_ln_h12288": base(s_local=3, b=3, h=12288, shard_index=2, t=8),
    "bf16_ln_h25600": base(s_local=5, b=1, h=25600, shard_index=7, t=8),
    "bf16_ln_h1000_ragged_wave_rows": base(s_local=37, b=1, h=1000),
    "bf16_ln_h2056_ragged_wg_row": base(s_local=7, b=2, h=2056),
    "fp32_ln_h260_ragged": base(s_local=13, b=3, h=260, io=F32),
    "fp32_rms_h3076_ragged": base(s_local=6, b=2, h=3076, io=F32, norm=RMS, p=0.3),
    "bf16_ln_h8_single_vector": base(s_local=5, b=1, h=8, p=0.5),
    "fp32_ln_h4_single_vector": base(s_local=9, b=1, h=4, io=F32, p=0.5),
    "bf16_ln_h32768_widest": base(s_local=2, b=1, h=32768),
    "fp32_ln_h16384_widest": base(s_local=2, b=1, h=16384, io=F32),
    "bf16_ln_one_row": base(s_local=1, b=1, h=6144),
    "bf16_ln_h6144_1003_rows": base(s_local=1003, b=1, h=6144),
    "fp32_ln_h256_1001_rows": base(s_local=1001, b=1, h=256, io=F32),
    "bf16_ln_high_counter_words": base(s_local=2, b=1, h=32768, shard_index=2**20 - 1,
                                       t=2**20, seed=2**64 - 1, offset=2**63 + 5),
    "bf16_ln_p0.9": base(s_local=4, b=2, h=6144, p=0.9),
    "fp32_ln_h8192_1100_rows": base(s_local=550, b=2, h=8192, io=F32),
    "bf16_rms_h12288_1500_rows": base(s_local=500, b=3, h=12288, norm=RMS, p=0.2),
    # 378 vectors: six per thread over 64-thread teams, six slots idle (ragged)
    "bf16_ln_h3024_ragged_six": base(s_local=9, b=2, h=3024),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_shapes(name):
    run_case(name, SMALL[name], seed=zlib.crc32(name.encode()) % 1000, with_dh_out=True,
             paths=(None, "fused", "split"), fwd_paths=(None, "rows", "stream"))


# Rows per tile of the split path's second pass and of the exit (16 and 32
# by default): other tilings must give results within the same tolerances,
# on shapes whose last tile is ragged.
@pytest.mark.parametrize("tile_rows", [16, 48, 64])
def test_split_tile_rows(tile_rows):
    run_case(f"split tiles of {tile_rows} rows", base(s_local=1003, b=1, h=6144, offset=3),
             seed=11, with_dh_out=True, paths=("split",), tile_rows=tile_rows)
    run_case(f"split tiles of {tile_rows} rows, fp32 RMS",
             base(s_local=37, b=3, h=3076, io=F32, norm=RMS, p=0.3), seed=12,
             paths=("split",), tile_rows=tile_rows)


@pytest.mark.parametrize("tile_rows", [32, 64])
def test_norm_free_exit_tile_rows(tile_rows):
    test_norm_free_exit("bf16_h8192_1100_rows", tile_rows)
    test_norm_free_exit("fp32_h260_ragged_p0.3", tile_rows)


# Seeded random shapes: widths anywhere in the supported range (bf16: any
# multiple of 8 up to 32768; fp32: of 4 up to 16384), 1-300 rows, either
# norm, several p, any shard of any t -- the launch plans' corner cases
# (ragged teams, wave rows, split backward) met at widths no list names.
def _random_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = {}
    while len(cases) < n:
        io = F32 if len(cases) % 3 == 2 else BF16
        epv = 8 if io == BF16 else 4
        hmax = 32768 if io == BF16 else 16384
        h = int(epv * rng.integers(1, hmax // epv + 1)) if rng.random() < 0.5 else \
            int(epv * np.exp(rng.uniform(0.0, np.log(hmax // epv))))
        h = max(epv, min(hmax, h - h % epv))
        rows = int(rng.integers(1, 301))
        rows = max(1, min(rows, 3_000_000 // h))
        b = int(rng.integers(1, 4))
        s_local = max(1, rows // b)
        t = int(rng.integers(1, 9))
        norm = LN if len(cases) % 2 == 0 else RMS
        p = float(rng.choice([0.0, 0.1, 0.5]))
        kw = base(s_local=s_local, b=b, h=h, io=io, norm=norm, p=p, t=t,
                  shard_index=int(rng.integers(0, t)), seed=int(rng.integers(0, 2**32)),
                  offset=int(rng.integers(0, 2**20)), eps=1e-5 if norm == LN else 1e-6)
        cases[f"{'bf16' if io == BF16 else 'fp32'}_{'ln' if norm == LN else 'rms'}_h{h}_"
              f"{s_local}x{b}_p{p}_t{t}"] = kw
    return cases


RANDOM = _random_cases()


@pytest.mark.parametrize("name", sorted(RANDOM))
def test_random_shapes(name):
    run_case(name, RANDOM[name], seed=zlib.crc32(name.encode()) % 1000,
             with_dh_out=bool(zlib.crc32(name.encode()) & 1))


# The mask-free region: the forward stores no mask and the backward
# regenerates the decisions from the same generator words.
MASK_FREE = {
    "bf16_ln_h6144_fused": (base(s_local=40, b=2, h=6144, shard_index=3, t=8), "fused"),
    "bf16_ln_h6144_split": (base(s_local=40, b=2, h=6144, shard_index=3, t=8), "split"),
    "bf16_ln_h25600_split": (base(s_local=3, b=2, h=25600, shard_index=1, t=4), None),
    "bf16_rms_h1000_wave_rows": (base(s_local=37, b=1, h=1000, norm=RMS, eps=1e-6), None),
    "fp32_ln_h3076_ragged": (base(s_local=6, b=2, h=3076, io=F32, p=0.3), None),
    "bf16_ln_h8192_1100_rows_stream": (base(s_local=1100, b=1, h=8192, offset=7), None),
}


@pytest.mark.parametrize("name", sorted(MASK_FREE))
def test_mask_free_region(name):
    kw, path = MASK_FREE[name]
    d, od = descs(**kw)
    _say(f"[case] mask-free {name}: {kw} bwd path {path or 'auto'}")
    inp = make_inputs(d.rows, d.h, d.io, seed=zlib.crc32(name.encode()) % 1000, dh_out=True)
    want = P.oracle_fwd(od, inp)
    with_mask = P.gpu_fwd(d, inp)
    no_mask = P.gpu_fwd(d, inp, store_mask=False)
    assert no_mask["mask"] is None
    P.check_fwd(dict(no_mask, mask=with_mask["mask"]), want, d.io)
    for k in ("h", "y", "mean", "rstd"):
        if want[k] is not None:
            P.exact(f"{k} (no mask stored vs stored)", no_mask[k], with_mask[k])
    wb = P.oracle_bwd(od, inp, want, True, True)
    regen = P.gpu_bwd(d, inp, dict(want, mask=None), with_dh_out=True, repeat=2, path=path)
    P.check_bwd(regen, wb, d.io)
    stored = P.gpu_bwd(d, inp, want, with_dh_out=True, path=path)
    for k in ("dx", "dres", "dgamma", "dbeta", "dbias"):
        if stored.get(k) is not None:
            P.exact(f"{k} (regenerated vs stored mask)", regen[k], stored[k])


# The reduce-scatter prologue: x is the sum of nparts partial slabs, added
# in the forward kernel.
RS = {
    "bf16_ln_h6144_t8": (base(s_local=16, b=4, h=6144, shard_index=3, t=8), 8),
    "bf16_ln_h6144_ring_last_step": (base(s_local=16, b=4, h=6144, shard_index=3, t=8), 2),
    "bf16_ln_h6144_one_part": (base(s_local=16, b=4, h=6144, shard_index=3, t=8), 1),
    "bf16_rms_h8192_5_parts": (base(s_local=20, b=1, h=8192, norm=RMS, eps=1e-6), 5),
    "fp32_ln_h260_ragged_3_parts": (base(s_local=13, b=3, h=260, io=F32), 3),
    "bf16_ln_h25600_t2": (base(s_local=3, b=2, h=25600, shard_index=1, t=2), 2),
    "bf16_ln_h3024_ragged_3_parts": (base(s_local=9, b=2, h=3024), 3),
    "bf16_ln_h32768_widest_9_parts": (base(s_local=2, b=1, h=32768), 9),
    "bf16_ln_h8192_1100_rows_t4": (base(s_local=1100, b=1, h=8192, t=4, shard_index=2), 4),
    "bf16_ln_h1000_wave_rows_p0_6_parts": (base(s_local=37, b=1, h=1000, p=0.0), 6),
}


@pytest.mark.parametrize("name", sorted(RS))
def test_reduce_scatter_prologue(name):
    kw, nparts = RS[name]
    d, od = descs(**kw)
    seed = zlib.crc32(name.encode()) % 1000
    _say(f"[case] reduce-scatter prologue {name}: {kw} nparts={nparts}")
    inp = make_inputs(d.rows, d.h, d.io, seed=seed)
    parts = make_parts(d.rows, d.h, d.io, nparts, seed=seed)
    x = oracle.reduce_parts(od, parts)
    want = P.oracle_fwd(od, dict(inp, x=x))
    # the row kernel on both sides (with one part, a stream-kernel choice
    # would otherwise send the prologue call to the stream kernel, whose
    # reductions run in another order)
    got = P.gpu_fwd_rs(P.tuned(d, fwd="rows"), inp, parts, nparts)
    P.check_fwd(got, want, d.io)
    # bit-identical to the plain forward (same kernel) on the summed x
    plain = P.gpu_fwd(d, dict(inp, x=x), path="rows")
    for k in ("h", "y", "mask", "mean", "rstd"):
        if plain[k] is not None:
            P.exact(f"{k} (fused prologue vs summed x)", got[k], plain[k])


# The two ends of the layer stack: the norm-only entry (no x: h is the
# residual) and the norm-free exit (no gamma: h and the mask only).
ENTRY = {
    "bf16_ln_h6144": base(s_local=16, b=4, h=6144, p=0.0),
    "fp32_rms_h3076_ragged": base(s_local=6, b=2, h=3076, io=F32, norm=RMS, p=0.0, eps=1e-6),
    "bf16_ln_h1000_wave_rows": base(s_local=37, b=1, h=1000, p=0.0),
    "bf16_rms_h8192_1100_rows": base(s_local=1100, b=1, h=8192, norm=RMS, p=0.0, eps=1e-6),
    "bf16_ln_h25600": base(s_local=3, b=2, h=25600, p=0.0),
    "bf16_ln_h3024_ragged": base(s_local=9, b=2, h=3024, p=0.0),
}


@pytest.mark.parametrize("name", sorted(ENTRY))
def test_norm_only_entry(name):
    import torch
    d, od = descs(**ENTRY[name])
    _say(f"[case] norm-only entry {name}: {ENTRY[name]}")
    inp = make_inputs(d.rows, d.h, d.io, seed=zlib.crc32(name.encode()) % 1000, dh_out=True)
    ln = d.norm == LN
    want = oracle.fwd(od, None, None, inp["residual"], inp["gamma"], inp["beta"] if ln else None)
    res = P.to_device(inp["residual"], d.io)
    gam, bet = P.to_device(inp["gamma"]), P.to_device(inp["beta"]) if ln else None
    for fpath in (None, "rows", "stream"):
        o = spr.fwd(P.tuned(d, fwd=fpath), None, None, res, gam, bet, write_h=False)
        oh = spr.fwd(P.tuned(d, fwd=fpath), None, None, res, gam, bet, write_h=True)
        got = {k: P.to_host(v) for k, v in o.items()}
        assert got["h"] is None and got["mask"] is None
        P.io_close("y", got["y"], want["y"], d.io)
        if ln:
            P.stats_close("mean", got["mean"], want["mean"])
        P.stats_close("rstd", got["rstd"], want["rstd"])
        P.exact("h (entry) = residual", P.to_host(oh["h"]), inp["residual"])
        for k in ("y", "mean", "rstd"):
            if got[k] is not None:
                P.exact(f"{k} (with and without h)", P.to_host(oh[k]), got[k])
    wb = oracle.bwd(od, inp["dy"], inp["dh_out"], inp["residual"], None, want["mean"],
                    want["rstd"], inp["gamma"], want_dbias=False, want_dx=False)
    for path in ("fused", "split"):
        dp = P.tuned(d, bwd=path)
        b = spr.alloc_bwd_outputs(dp, res.device, want_dbias=False)
        spr.sp_region_bwd(dp, P.to_device(inp["dy"], d.io), P.to_device(inp["dh_out"], d.io),
                          res, None, P.to_device(want["mean"]), P.to_device(want["rstd"]),
                          gam, None, b["dres"], b["dgamma"], b["dbeta"], None,
                          b["workspace"])
        torch.cuda.synchronize()
        P.io_close(f"dres ({path})", P.to_host(b["dres"]), wb["dres"], d.io)
        P.param_grad_close(f"dgamma ({path})", P.to_host(b["dgamma"]), wb["dgamma"])
        if ln:
            P.param_grad_close(f"dbeta ({path})", P.to_host(b["dbeta"]), wb["dbeta"])


EXIT = {
    "bf16_h6144_p0.1_shard2of4": base(s_local=16, b=4, h=6144, shard_index=2, t=4),
    "fp32_h260_ragged_p0.3": base(s_local=13, b=3, h=260, io=F32, p=0.3),
    "bf16_h25600_p0": base(s_local=3, b=2, h=25600, p=0.0),
    "bf16_h8192_1100_rows": base(s_local=1100, b=1, h=8192, offset=5),
    "fp32_h4_single_vector": base(s_local=9, b=1, h=4, io=F32, p=0.5),
    "bf16_h3024_ragged_p0.1": base(s_local=9, b=2, h=3024),
}


@pytest.mark.parametrize("name", sorted(EXIT))
def test_norm_free_exit(name, tile_rows=None):
    import torch
    d, od = descs(**EXIT[name])
    d = P.tuned(d, tile_rows=tile_rows)
    _say(f"[case] norm-free exit {name}: {EXIT[name]}")
    inp = make_inputs(d.rows, d.h, d.io, seed=zlib.crc32(name.encode()) % 1000, dh_out=True)
    want = oracle.fwd(od, inp["x"], inp["bias"], inp["residual"], None, None)
    x, res = P.to_device(inp["x"], d.io), P.to_device(inp["residual"], d.io)
    bias = P.to_device(inp["bias"])
    for fpath in (None, "rows", "stream"):
        o = spr.fwd(P.tuned(d, fwd=fpath), x, bias, res, None, None)
        got = {k: P.to_host(v) for k, v in o.items()}
        for k in ("y", "mean", "rstd"):
            assert got[k] is None
        P.exact("h (exit)", got["h"], want["h"])
        if want["mask"] is not None:
            P.exact("mask (exit)", got["mask"], want["mask"])
    wb = oracle.bwd(od, None, inp["dh_out"], None, want["mask"], None, None, None,
                    want_dres=False)
    dho = P.to_device(inp["dh_out"], d.io)
    results = []
    for mask in ((want["mask"], None) if d.p > 0 else (None,)):
        for with_dbias in (True, False):
            dx = torch.empty_like(dho)
            dbias = torch.empty(d.h, dtype=torch.float32, device=dho.device) if with_dbias else None
            ws = torch.zeros(max(spr.sp_region_bwd_workspace_bytes(d), 16), dtype=torch.uint8,
                             device=dho.device) if with_dbias else None
            spr.sp_region_bwd_exit(d, dho, P.to_device(mask), dx, dbias, ws)
            torch.cuda.synchronize()
            gdx = P.to_host(dx)
            P.io_close("dx (exit)", gdx, wb["dx"], d.io)
            if with_dbias:
                P.param_grad_close("dbias (exit)", P.to_host(dbias), wb["dbias"])
            results.append(gdx)
    for r in results[1:]:
        P.exact("dx (exit; mask stored vs regenerated, dbias or not)", r, results[0])


@pytest.mark.parametrize("with_bias,with_dh_out,want_dbias", [(False, False, True),
                                                              (True, False, False),
                                                              (False, True, False)])
@pytest.mark.parametrize("io,norm", [(BF16, LN), (F32, RMS)])
def test_optional_arguments(with_bias, with_dh_out, want_dbias, io, norm):
    kw = base(s_local=6, b=2, h=6144 if io == BF16 else 1024, io=io, norm=norm)
    run_case(f"optional io={io} norm={norm}", kw, seed=3, with_bias=with_bias,
             with_dh_out=with_dh_out, want_dbias=want_dbias, paths=("fused", "split"))


def test_tiny_fp32_workload_as_specified():
    """The tiny fp32 workload exactly as specified: the full [128, 2, 256]
    tensor (seed 0, x, residual and the gradient of y standard normal, bias
    and beta N(0, 0.02), gamma 1 + N(0, 0.02); LayerNorm eps 1e-5, p 0.1),
    run unsharded (t = 1) and as both shards [64, 2, 256] of t = 2.  Each
    run is checked element by element against the oracle; the two shards
    concatenated equal the t = 1 run bit for bit (the band is per token:
    "Sequence parallel math", section "The move: split the LayerNorm/dropout
    band along the sequence"), and the shards' parameter gradients summed
    equal the t = 1 ones within 1e-4."""
    w = WORKLOADS["tiny_fp32_t2"]
    full_kw = dict(s_local=w.s, b=w.b, h=w.h, shard_index=0, t=1, io=w.io, norm=w.norm, p=w.p,
                   eps=w.eps, seed=w.seed, offset=0)
    full, ofull = descs(**full_kw)
    _say(f"[case] tiny fp32 workload, unsharded: {full_kw}")
    inp = make_inputs(full.rows, w.h, w.io, seed=w.seed)
    want = P.oracle_fwd(ofull, inp)
    ref = P.gpu_fwd(full, inp)
    P.check_fwd(ref, want, w.io)
    wantb = P.oracle_bwd(ofull, inp, want)
    refb = P.gpu_bwd(full, inp, ref, repeat=2)
    P.check_bwd(refb, wantb, w.io)
    N = w.rows
    acc = {k: np.zeros(w.h) for k in ("dgamma", "dbeta", "dbias")}
    for i in range(w.t):
        kw = dict(full_kw, s_local=w.s_local, shard_index=i, t=w.t)
        d, od = descs(**kw)
        _say(f"[case] tiny fp32 workload, shard {i} of {w.t}: {kw}")
        sl = slice(i * N * w.h, (i + 1) * N * w.h)
        si = {k: (v[sl] if v is not None and v.size == full.rows * w.h else v)
              for k, v in inp.items()}
        ws = P.oracle_fwd(od, si)
        o = P.gpu_fwd(d, si)
        P.check_fwd(o, ws, w.io)
        wbs = P.oracle_bwd(od, si, ws)
        g = P.gpu_bwd(d, si, o, repeat=2)
        P.check_bwd(g, wbs, w.io)
        for k in ("h", "y", "mask"):
            P.exact(f"{k} shard {i} vs t=1", o[k], ref[k][sl])
            P.exact(f"oracle {k} shard {i} vs t=1", ws[k], want[k][sl])
        for k in ("mean", "rstd"):
            P.exact(f"{k} shard {i} vs t=1", o[k], ref[k][i * N:(i + 1) * N])
        for k in ("dx", "dres"):
            P.exact(f"{k} shard {i} vs t=1", g[k], refb[k][sl])
        for k in acc:
            acc[k] += g[k]
    for k in acc:
        P.param_grad_close(f"sum of shard {k} vs t=1", acc[k], refb[k])


@pytest.mark.parametrize("io,h,t", [(F32, 256, 2), (BF16, 6144, 4), (BF16, 25600, 2)])
def test_shard_invariance(io, h, t):
    """Concatenating the t shard results equals the unsharded (t = 1) run:
    bit-exact for every per-token output, and the parameter gradients summed
    over shards match within tolerance."""
    s, b = 16, 2
    full, _ = descs(**base(s_local=s, b=b, h=h, io=io, t=1, offset=3))
    _say(f"[case] shard invariance io={io} h={h} t={t}")
    inp = make_inputs(full.rows, h, io, seed=11, dh_out=True)
    ref = P.gpu_fwd(full, inp)
    refb = P.gpu_bwd(full, inp, ref, with_dh_out=True)
    N = full.rows // t
    acc = {k: np.zeros(h) for k in ("dgamma", "dbeta", "dbias")}
    for i in range(t):
        d, _ = descs(**base(s_local=s // t, b=b, h=h, io=io, shard_index=i, t=t, offset=3))
        sl = slice(i * N * h, (i + 1) * N * h)
        si = {k: (v[sl] if v is not None and v.size == full.rows * h else v) for k, v in inp.items()}
        o = P.gpu_fwd(d, si)
        for k in ("h", "y", "mask"):
            P.exact(f"{k} shard {i}", o[k], ref[k][sl])
        for k in ("mean", "rstd"):
            P.exact(f"{k} shard {i}", o[k], ref[k][i * N:(i + 1) * N])
        g = P.gpu_bwd(d, si, o, with_dh_out=True)
        for k in ("dx", "dres"):
            P.exact(f"{k} shard {i}", g[k], refb[k][sl])
        for k in acc:
            acc[k] += g[k]
    for k in acc:
        P.param_grad_close(f"sum of shard {k}", acc[k], refb[k])


def test_workspace_and_argument_errors_leave_outputs_untouched():
    import torch
    d, _ = descs(**base(s_local=4, b=2, h=6144))
    inp = make_inputs(d.rows, d.h, d.io, seed=1)
    dev = "cuda:0"
    x, res = P.to_device(inp["x"], BF16), P.to_device(inp["residual"], BF16)
    g, bt = P.to_device(inp["gamma"]), P.to_device(inp["beta"])
    o = spr.alloc_fwd_outputs(d, dev)
    for v in o.values():
        v.view(torch.uint8).fill_(0xA5)
    bad = spr.Desc(**dict(base(s_local=4, b=2, h=6144), p=1.5))
    with pytest.raises(spr.SprError) as e:
        spr.sp_region_fwd(bad, x, None, res, g, bt, o["h"], o["y"], o["mask"], o["mean"], o["rstd"])
    assert e.value.status == spr.SPR_ERR_INVALID_ARG
    torch.cuda.synchronize()
    for v in o.values():
        assert bool((v.view(torch.uint8) == 0xA5).all())
    spr.sp_region_fwd(d, x, None, res, g, bt, o["h"], o["y"], o["mask"], o["mean"], o["rstd"])
    ob = spr.alloc_bwd_outputs(d, dev)
    small = ob["workspace"][:-256] if ob["workspace"].numel() > 256 else ob["workspace"][:0]
    with pytest.raises(spr.SprError) as e:
        spr.sp_region_bwd(d, x, None, o["h"], o["mask"], o["mean"], o["rstd"], g, ob["dx"],
                          ob["dres"], ob["dgamma"], ob["dbeta"], ob["dbias"], small)
    assert e.value.status == spr.SPR_ERR_WORKSPACE


@pytest.mark.parametrize("path", ["fused", "split"])
def test_launch_by_launch_equals_whole_backward(path):
    """Running the backward's launches one at a time on the stream gives the
    same bits as sp_region_bwd."""
    import torch
    d, od = descs(**base(s_local=37, b=2, h=6144))
    d = P.tuned(d, bwd=path)
    _say(f"[case] launch by launch, path {path}")
    inp = make_inputs(d.rows, d.h, d.io, seed=4, dh_out=True)
    saved = P.oracle_fwd(od, inp)
    args = (P.to_device(inp["dy"], d.io), P.to_device(inp["dh_out"], d.io),
            P.to_device(saved["h"], d.io), P.to_device(saved["mask"]), P.to_device(saved["mean"]),
            P.to_device(saved["rstd"]), P.to_device(inp["gamma"]))
    whole = spr.alloc_bwd_outputs(d, "cuda:0")
    spr.sp_region_bwd(d, *args, whole["dx"], whole["dres"], whole["dgamma"], whole["dbeta"],
                      whole["dbias"], whole["workspace"])
    parts = spr.alloc_bwd_outputs(d, "cuda:0")
    n = spr.sp_region_bwd_num_launches(d)
    assert n == (2 if path == "fused" else 3)
    for i in range(n):
        spr.sp_region_bwd_launch(d, i, *args, parts["dx"], parts["dres"], parts["dgamma"],
                                 parts["dbeta"], parts["dbias"], parts["workspace"])
    torch.cuda.synchronize()
    for k in ("dx", "dres", "dgamma", "dbeta", "dbias"):
        P.exact(k, P.to_host(parts[k]), P.to_host(whole[k]))


def test_outputs_stay_inside_their_buffers():
    """Every output is a view into a larger buffer whose guard bands hold a
    pattern; after fwd and bwd the guards are unchanged."""
    import torch
    G = 256                                   # guard elements (keeps 16-byte alignment)
    for kw in (base(s_local=7, b=3, h=2056), base(s_local=9, b=1, h=260, io=F32),
               base(s_local=3, b=1, h=25600)):
        d, _ = descs(**kw)
        _say(f"[case] guards {kw}")
        inp = make_inputs(d.rows, d.h, d.io, seed=2, dh_out=True)
        dev = "cuda:0"

        def guarded(n, dtype):
            full = torch.empty(n + 2 * G, dtype=dtype, device=dev)
            full.view(torch.uint8).fill_(0x5A)
            return full, full[G:G + n]

        io = torch.bfloat16 if d.io == BF16 else torch.float32
        N, H = d.rows, d.h
        bufs = {k: guarded(n, dt) for k, (n, dt) in {
            "h": (N * H, io), "y": (N * H, io), "mask": (N * H, torch.uint8),
            "mean": (N, torch.float32), "rstd": (N, torch.float32), "dx": (N * H, io),
            "dres": (N * H, io), "dgamma": (H, torch.float32), "dbeta": (H, torch.float32),
            "dbias": (H, torch.float32),
            "ws": (spr.sp_region_bwd_workspace_bytes(d) // 4, torch.float32)}.items()}
        v = {k: b[1] for k, b in bufs.items()}
        v["ws"].zero_()
        spr.sp_region_fwd(d, P.to_device(inp["x"], d.io), P.to_device(inp["bias"]),
                          P.to_device(inp["residual"], d.io), P.to_device(inp["gamma"]),
                          P.to_device(inp["beta"]), v["h"], v["y"], v["mask"], v["mean"], v["rstd"])
        spr.sp_region_bwd(d, P.to_device(inp["dy"], d.io), P.to_device(inp["dh_out"], d.io),
                          v["h"], v["mask"], v["mean"], v["rstd"], P.to_device(inp["gamma"]),
                          v["dx"], v["dres"], v["dgamma"], v["dbeta"], v["dbias"], v["ws"])
        torch.cuda.synchronize()
        for k, (full, _) in bufs.items():
            raw = full.view(torch.uint8)
            gb = G * full.element_size()
            assert bool((raw[:gb] == 0x5A).all()) and bool((raw[-gb:] == 0x5A).all()), k


# ------------------------------------------------------------------ full size
def _full_kw(w, shard_index=0, offset=0):
    return dict(s_local=w.s_local, b=w.b, h=w.h, shard_index=shard_index, t=w.t, io=w.io,
                norm=w.norm, p=w.p, eps=w.eps, seed=w.seed, offset=offset)


@pytest.mark.parametrize("name", ["22b_h6144_t8", "longseq_rms_h8192_t8_p0.1",
                                  "longseq_rms_h8192_t8_p0", "1t_h25600_t8", "1t_h25600_t4",
                                  "1t_h25600_t2", "1t_h25600_t1"])
def test_full_size_workload(name):
    """The workloads at their real shard shapes, in the launch configuration
    the benchmark times; every element is compared."""
    w = WORKLOADS[name]
    run_case(name, _full_kw(w), seed=w.seed, with_dh_out=(w.norm == RMS),
             paths=(None, "fused", "split"))


def test_full_size_175b_layer_two_calls():
    """175B-class layer: the pre-attention and pre-MLP region calls chained
    as in a layer (call B's residual is call A's h; call A's backward gets
    call B's dresidual as dh_out), offsets 0 and 1 for the two dropout sites."""
    w = WORKLOADS["175b_h12288_t8"]
    dA, odA = descs(**_full_kw(w, offset=0))
    dB, odB = descs(**_full_kw(w, offset=1))
    _say(f"[case] 175b layer: {_full_kw(w)}")
    inA = make_inputs(dA.rows, dA.h, dA.io, seed=0)
    inB = make_inputs(dB.rows, dB.h, dB.io, seed=1)
    # forward: A then B, B's residual = A's h
    wA = P.oracle_fwd(odA, inA)
    gA = P.gpu_fwd(dA, inA)
    P.check_fwd(gA, wA, dA.io)
    inB_o = dict(inB, residual=wA["h"])
    wB = P.oracle_fwd(odB, inB_o)
    gB = P.gpu_fwd(dB, dict(inB, residual=gA["h"]))
    P.check_fwd(gB, wB, dB.io)
    # backward: B then A, A's dh_out = B's dresidual
    wbB = P.oracle_bwd(odB, inB_o, wB)
    gbB = P.gpu_bwd(dB, inB_o, wB)
    P.check_bwd(gbB, wbB, dB.io)
    inA_b = dict(inA, dh_out=wbB["dres"])
    wbA = P.oracle_bwd(odA, inA_b, wA, with_dh_out=True)
    gbA = P.gpu_bwd(dA, inA_b, wA, with_dh_out=True)
    P.check_bwd(gbA, wbA, dA.io)

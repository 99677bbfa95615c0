"""Comparison rules between the GPU library and the CPU oracle.

Bit-exact: the dropout mask and h (a fixed sequence of IEEE fp32 operations
and one round-to-nearest-even).  Tolerances for the rest, with fp32
accumulation on the GPU and float64 in the oracle:
  y            fp32 I/O: max |a - b| <= 1e-5
               bf16 I/O: |a - b| <= ulp_bf16(b) + 1e-3 per element
  mean, rstd   |a - b| <= 1e-5 * |b| (+ 1e-6 absolute for means near 0)
  dx, dres     fp32 I/O: max|a - b| / max|b| <= 1e-4
               bf16 I/O: |a - b| <= ulp_bf16(b) + 1e-3 per element
  dgamma, dbeta, dbias (fp32): max|a - b| / max|b| <= 1e-4
ulp_bf16(b) = 2^(floor(log2 |b|) - 7), the spacing of bfloat16 at b.
"""
import numpy as np

F32, BF16 = 0, 1


def widen(a, io):
    """I/O array (float32, or uint16 bf16 bits) -> float64."""
    if io == BF16:
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


def ulp_bf16(b):
    b = np.abs(b)
    e = np.floor(np.log2(np.where(b > 0, b, 1.0)))
    return np.where(b > 0, np.exp2(e - 7), 0.0)


def _fail(name, msg):
    raise AssertionError(f"{name}: {msg}")


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view({1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[a.dtype.itemsize])


def exact(name, got, want):
    got, want = np.asarray(got), np.asarray(want)
    if got.shape != want.shape or got.dtype != want.dtype:
        _fail(name, f"shape/dtype {got.shape} {got.dtype} vs {want.shape} {want.dtype}")
    bad = np.flatnonzero(_bits(got) != _bits(want))
    if bad.size:
        i = bad[0]
        _fail(name, f"{bad.size} of {got.size} differ; first at {i}: {got.flat[i]} vs {want.flat[i]}")


def io_close(name, got, want, io):
    """y, dx, dres rule."""
    a, b = widen(got, io), widen(want, io)
    if io == F32:
        err = np.max(np.abs(a - b)) if a.size else 0.0
        if name in ("dx", "dres"):
            ref = np.max(np.abs(b)) if b.size else 1.0
            if err > 1e-4 * max(ref, 1e-30):
                _fail(name, f"norm-wise rel err {err / ref:.3e} > 1e-4")
        elif err > 1e-5:
            _fail(name, f"max abs err {err:.3e} > 1e-5")
        return
    tol = ulp_bf16(b) + 1e-3
    bad = np.flatnonzero(np.abs(a - b) > tol)
    if bad.size:
        i = bad[0]
        _fail(name, f"{bad.size} of {a.size} outside ulp+1e-3; first at {i}: {a[i]} vs {b[i]}")


def stats_close(name, got, want):
    a, b = np.asarray(got, np.float64), np.asarray(want, np.float64)
    bad = np.flatnonzero(np.abs(a - b) > 1e-5 * np.abs(b) + 1e-6)
    if bad.size:
        i = bad[0]
        _fail(name, f"{bad.size} rows off; first at {i}: {a[i]} vs {b[i]}")


def param_grad_close(name, got, want):
    a, b = np.asarray(got, np.float64), np.asarray(want, np.float64)
    ref = np.max(np.abs(b))
    err = np.max(np.abs(a - b))
    if err > 1e-4 * max(ref, 1e-30):
        _fail(name, f"norm-wise rel err {err / ref:.3e} > 1e-4")


def check_fwd(got, want, io):
    if want["mask"] is not None:
        exact("mask", got["mask"], want["mask"])
    exact("h", got["h"], want["h"])
    io_close("y", got["y"], want["y"], io)
    if want["mean"] is not None:
        stats_close("mean", got["mean"], want["mean"])
    stats_close("rstd", got["rstd"], want["rstd"])


def check_bwd(got, want, io):
    io_close("dx", got["dx"], want["dx"], io)
    io_close("dres", got["dres"], want["dres"], io)
    for k in ("dgamma", "dbeta", "dbias"):
        if want.get(k) is not None:
            param_grad_close(k, got[k], want[k])


# ------------------------------------------------------------------ runners
def to_device(a, io=None, device="cuda:0"):
    """numpy -> torch on the GPU; uint16 arrays with io == BF16 become bfloat16."""
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if io == BF16 and a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


def to_host(t):
    """torch (GPU) -> numpy; bfloat16 becomes uint16 bits."""
    import torch
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oracle_fwd(od, inp, with_bias=True, rows=None):
    import oracle
    sl = slice(None) if rows is None else slice(rows[0] * od.h, rows[1] * od.h)
    return oracle.fwd(od, inp["x"][sl], inp["bias"] if with_bias else None, inp["residual"][sl],
                      inp["gamma"], inp["beta"] if od.norm == 0 else None, rows=rows)


def oracle_bwd(od, inp, saved, with_dh_out=False, want_dbias=True):
    import oracle
    return oracle.bwd(od, inp["dy"], inp["dh_out"] if with_dh_out else None, saved["h"],
                      saved["mask"], saved["mean"], saved["rstd"], inp["gamma"],
                      want_dbias=want_dbias)


_FWD = {None: 0, "rows": 1, "stream": 2}
_BWD = {None: 0, "fused": 1, "split": 2}


def tuned(d, fwd=None, bwd=None, tile_rows=None):
    """d with the launch choices set: fwd = "rows" or "stream" (forward
    kernel), bwd = "fused" or "split" (backward path), tile_rows (split and
    exit tiles); None leaves a choice to the library."""
    import dataclasses
    kw = {}
    if fwd is not None:
        kw["fwd_kernel"] = _FWD[fwd]
    if bwd is not None:
        kw["bwd_path"] = _BWD[bwd]
    if tile_rows is not None:
        kw["bwd_tile_rows"] = int(tile_rows)
    return dataclasses.replace(d, **kw) if kw else d


def gpu_fwd(d, inp, with_bias=True, device="cuda:0", path=None, store_mask=True):
    """Forward on the GPU; path = "rows" or "stream" asks the library for
    that forward kernel, None for its own choice.
    store_mask=False: no mask is stored (the backward regenerates it)."""
    import dropout_region_amd as spr
    io = d.io
    o = spr.fwd(tuned(d, fwd=path), to_device(inp["x"], io, device),
                to_device(inp["bias"], device=device) if with_bias else None,
                to_device(inp["residual"], io, device), to_device(inp["gamma"], device=device),
                to_device(inp["beta"], device=device) if d.norm == 0 else None,
                store_mask=store_mask)
    return {k: to_host(v) for k, v in o.items()}


def gpu_fwd_rs(d, inp, parts, nparts, with_bias=True, device="cuda:0"):
    """sp_region_fwd_rs on the GPU: x is the sum of the nparts slabs `parts`."""
    import dropout_region_amd as spr
    io = d.io
    o = spr.fwd_rs(d, to_device(np.ascontiguousarray(parts).ravel(), io, device), nparts,
                   to_device(inp["bias"], device=device) if with_bias else None,
                   to_device(inp["residual"], io, device), to_device(inp["gamma"], device=device),
                   to_device(inp["beta"], device=device) if d.norm == 0 else None)
    return {k: to_host(v) for k, v in o.items()}


def gpu_bwd(d, inp, saved, with_dh_out=False, want_dbias=True, device="cuda:0", repeat=1,
            path=None):
    """Backward from `saved` (host arrays of h, mask, mean, rstd).  With
    repeat > 1 the call is made that many times into the same outputs and
    workspace, and every result must be bit-identical.  path = "fused" or
    "split" asks the library for that backward path."""
    import dropout_region_amd as spr
    return _gpu_bwd(spr, tuned(d, bwd=path), inp, saved, with_dh_out, want_dbias, device, repeat)


def _gpu_bwd(spr, d, inp, saved, with_dh_out, want_dbias, device, repeat):
    io = d.io
    args = (to_device(inp["dy"], io, device),
            to_device(inp["dh_out"], io, device) if with_dh_out else None,
            to_device(saved["h"], io, device), to_device(saved["mask"], device=device),
            to_device(saved["mean"], device=device), to_device(saved["rstd"], device=device),
            to_device(inp["gamma"], device=device))
    o = spr.alloc_bwd_outputs(d, device, want_dbias)
    first = None
    for _ in range(repeat):
        spr.sp_region_bwd(d, *args, o["dx"], o["dres"], o["dgamma"], o["dbeta"], o["dbias"],
                          o["workspace"])
        res = {k: to_host(v) for k, v in o.items() if k != "workspace"}
        if first is None:
            first = res
        else:
            for k, v in res.items():
                if v is not None:
                    exact(f"{k} (repeat)", v, first[k])
    return first

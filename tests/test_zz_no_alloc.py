"""sp_region_bwd_noalloc (the backward with the library's fixed scratch, for
callers that cannot allocate) against sp_region_bwd with a workspace of its
own: the same kernels, so the same bits.  Two calls in a row on each
backward path, the second on a smaller shard, so the second call runs over
scratch the first one left behind; every result is also checked against the
oracle."""
import numpy as np
import pytest

import dropout_region_amd as spr
import oracle
from sp_inputs import make_inputs
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    spr.lib()


def _run(kw, seed, path):
    import torch
    d, od = spr.Desc(**kw), oracle.Desc(**kw)
    d = P.tuned(d, bwd=path)
    _say(f"[case] no-alloc backward {path}: {kw}")
    inp = make_inputs(d.rows, d.h, d.io, seed=seed, dh_out=True)
    saved = P.oracle_fwd(od, inp)
    args = (P.to_device(inp["dy"], d.io), P.to_device(inp["dh_out"], d.io),
            P.to_device(saved["h"], d.io), P.to_device(saved["mask"]),
            P.to_device(saved["mean"]) if saved["mean"] is not None else None,
            P.to_device(saved["rstd"]), P.to_device(inp["gamma"]))
    ref = spr.alloc_bwd_outputs(d, "cuda:0")
    spr.sp_region_bwd(d, *args, ref["dx"], ref["dres"], ref["dgamma"], ref["dbeta"], ref["dbias"],
                      ref["workspace"])
    got = spr.alloc_bwd_outputs(d, "cuda:0")
    spr.sp_region_bwd_noalloc(d, *args, got["dx"], got["dres"], got["dgamma"], got["dbeta"],
                              got["dbias"])
    torch.cuda.synchronize()
    keys = [k for k in ("dx", "dres", "dgamma", "dbeta", "dbias") if ref[k] is not None]
    for k in keys:
        P.exact(f"{k} (no-alloc vs workspace)", P.to_host(got[k]), P.to_host(ref[k]))
    want = P.oracle_bwd(od, inp, saved, with_dh_out=True)
    P.check_bwd({k: P.to_host(got[k]) for k in keys}, want, d.io)


def _base(**kw):
    b = dict(shard_index=1, t=8, io=spr.SPR_BF16, norm=spr.SPR_LAYERNORM, p=0.1, eps=1e-5,
             seed=7, offset=2)
    b.update(kw)
    return b


@pytest.mark.parametrize("path", ["fused", "split"])
def test_no_alloc_backward_equals_the_workspace_backward(path):
    if path == "fused":
        # the 22B-class shard (256 partial rows of 3*6144 fp32), then a smaller one
        big = _base(s_local=256, b=4, h=6144)
        small = _base(s_local=5, b=3, h=6144, norm=spr.SPR_RMSNORM, eps=1e-6)
    else:
        big = _base(s_local=160, b=4, h=25600, shard_index=0, t=2)
        small = _base(s_local=7, b=2, h=3076, io=spr.SPR_F32, p=0.3)
    _run(big, 1, path)
    _run(small, 2, path)


"""The region as a torch autograd function (dropout_region_amd.region):
its gradients are those of the C ABI's backward called directly, bit for
bit, with dL/dy as dy and dL/dh as dh_out."""
import pytest

import dropout_region_amd as spr
from sp_inputs import make_inputs
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io,norm,with_bias", [(P.BF16, spr.SPR_LAYERNORM, True),
                                               (P.F32, spr.SPR_RMSNORM, False)])
def test_autograd_matches_direct_backward(io, norm, with_bias):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    d = spr.Desc(s_local=48, b=2, h=1536, shard_index=1, t=2, io=io, norm=norm, p=0.1, seed=5)
    print(f"[case] autograd region io={io} norm={norm} bias={with_bias}", flush=True)
    x = make_inputs(d.rows, d.h, io, seed=3, dh_out=True)
    dev = lambda a: P.to_device(a, io)
    xs, rs = dev(x["x"]).requires_grad_(), dev(x["residual"]).requires_grad_()
    bias = P.to_device(x["bias"], P.F32).requires_grad_() if with_bias else None
    gamma = P.to_device(x["gamma"], P.F32).requires_grad_()
    beta = P.to_device(x["beta"], P.F32).requires_grad_() if norm == spr.SPR_LAYERNORM else None
    y, h = spr.region(d, xs, rs, bias, gamma, beta)
    wy, wh = dev(x["dy"]), dev(x["dh_out"])
    # loss = <y, wy> + <h, wh>: dL/dy = wy and dL/dh = wh exactly
    loss = (y.double() * wy.double()).sum() + (h.double() * wh.double()).sum()
    loss.backward()
    torch.cuda.synchronize()

    o = spr.fwd(d, dev(x["x"]), None if bias is None else bias.detach(), dev(x["residual"]),
                gamma.detach(), None if beta is None else beta.detach())
    g = spr.bwd(d, wy, wh, o["h"], o["mask"], o["mean"], o["rstd"], gamma.detach(),
                want_dbias=with_bias)
    torch.cuda.synchronize()
    P.exact("y", P.to_host(y.detach()), P.to_host(o["y"]))
    P.exact("h", P.to_host(h.detach()), P.to_host(o["h"]))
    P.exact("dx", P.to_host(xs.grad), P.to_host(g["dx"]))
    P.exact("dresidual", P.to_host(rs.grad), P.to_host(g["dres"]))
    P.exact("dgamma", P.to_host(gamma.grad), P.to_host(g["dgamma"]))
    if beta is not None:
        P.exact("dbeta", P.to_host(beta.grad), P.to_host(g["dbeta"]))
    if bias is not None:
        P.exact("dbias", P.to_host(bias.grad), P.to_host(g["dbias"]))

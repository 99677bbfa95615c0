"""Pins of the oracle's two region variants at the ends of the layer stack.

Norm-only entry (x = None): the first block's LayerNorm/RMSNorm reads the
residual stream directly, with no branch before it, so h is the residual
bit for bit and y = Norm(residual).  Norm-free exit (gamma = None): the last
residual add with no norm after it, so the region is h = residual +
dropout(x + bias) and its backward takes dh = dh_out.

Pinned against torch float64 (layer_norm / rms_norm, autograd), exact
bit patterns (a negative zero survives the entry), and the full region
(identical h and mask)."""
import numpy as np
import pytest
import torch

import oracle
from sp_inputs import make_inputs

LN, RMS, F32, BF16 = oracle.LAYERNORM, oracle.RMSNORM, oracle.F32, oracle.BF16


def _widen(d, a):
    return np.asarray(a, np.float32) if d.io == F32 else oracle.bf16_to_f32(a)


# ------------------------------------------------------------ norm-only entry
@pytest.mark.parametrize("io", [F32, BF16])
def test_entry_h_is_the_residual_bit_for_bit(olib, io):
    d = oracle.Desc(s_local=4, b=2, h=64, io=io, norm=LN, p=0.0)
    inp = make_inputs(d.rows, d.h, io, seed=40)
    res = inp["residual"].copy()
    res[::7] = 0x8000 if io == BF16 else np.float32(-0.0)   # negative zeros: x + 0 would flip them
    out = oracle.fwd(d, None, None, res, inp["gamma"], inp["beta"], L=olib)
    assert out["mask"] is None
    assert np.array_equal(np.asarray(out["h"]).view(np.uint8), np.asarray(res).view(np.uint8))
    no_h = oracle.fwd(d, None, None, res, inp["gamma"], inp["beta"], L=olib, write_h=False)
    assert no_h["h"] is None
    for k in ("y", "mean", "rstd"):
        assert np.array_equal(no_h[k], out[k]), k


@pytest.mark.parametrize("norm", [LN, RMS])
def test_entry_y_is_torch_norm_of_the_residual(olib, norm):
    d = oracle.Desc(s_local=8, b=2, h=96, io=F32, norm=norm, p=0.0, eps=1e-5)
    inp = make_inputs(d.rows, d.h, F32, seed=41)
    beta = inp["beta"] if norm == LN else None
    out = oracle.fwd(d, None, None, inp["residual"], inp["gamma"], beta, L=olib)
    r64 = torch.from_numpy(inp["residual"].astype(np.float64).reshape(d.rows, d.h))
    g64 = torch.from_numpy(inp["gamma"].astype(np.float64))
    if norm == LN:
        ref = torch.nn.functional.layer_norm(r64, (d.h,), g64,
                                             torch.from_numpy(beta.astype(np.float64)), d.eps)
    else:
        ref = torch.nn.functional.rms_norm(r64, (d.h,), g64, d.eps)
    ref32 = ref.numpy().astype(np.float32).ravel()
    ulps = np.abs(out["y"].view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1


@pytest.mark.parametrize("norm", [LN, RMS])
def test_entry_backward_matches_torch_autograd(olib, norm):
    d = oracle.Desc(s_local=8, b=2, h=64, io=F32, norm=norm, p=0.0, eps=1e-5)
    inp = make_inputs(d.rows, d.h, F32, seed=42, dh_out=True)
    beta = inp["beta"] if norm == LN else None
    out = oracle.fwd(d, None, None, inp["residual"], inp["gamma"], beta, L=olib)
    g = oracle.bwd(d, inp["dy"], inp["dh_out"], inp["residual"], None, out["mean"], out["rstd"],
                   inp["gamma"], want_dbias=False, want_dx=False, L=olib)
    assert g["dx"] is None and g["dbias"] is None
    r = torch.tensor(inp["residual"].astype(np.float64).reshape(d.rows, d.h), requires_grad=True)
    gam = torch.tensor(inp["gamma"].astype(np.float64), requires_grad=True)
    bet = torch.tensor(beta.astype(np.float64), requires_grad=True) if norm == LN else None
    if norm == LN:
        y = torch.nn.functional.layer_norm(r, (d.h,), gam, bet, d.eps)
    else:
        y = torch.nn.functional.rms_norm(r, (d.h,), gam, d.eps)
    dy = torch.from_numpy(inp["dy"].astype(np.float64).reshape(d.rows, d.h))
    dho = torch.from_numpy(inp["dh_out"].astype(np.float64).reshape(d.rows, d.h))
    ((y * dy).sum() + (r * dho).sum()).backward()
    ref = {"dres": r.grad.numpy().ravel(), "dgamma": gam.grad.numpy()}
    if norm == LN:
        ref["dbeta"] = bet.grad.numpy()
    for k, v in ref.items():
        rel = np.max(np.abs(g[k].astype(np.float64) - v)) / np.max(np.abs(v))
        assert rel <= 1e-5, (k, rel)


# ------------------------------------------------------------ norm-free exit
@pytest.mark.parametrize("io", [F32, BF16])
def test_exit_h_and_mask_are_the_full_regions(olib, io):
    d = oracle.Desc(s_local=6, b=2, h=80, io=io, norm=LN, p=0.25, shard_index=1, t=3, seed=9)
    inp = make_inputs(d.rows, d.h, io, seed=43)
    full = oracle.fwd(d, inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"],
                      L=olib)
    ex = oracle.fwd(d, inp["x"], inp["bias"], inp["residual"], None, None, L=olib)
    for k in ("y", "mean", "rstd"):
        assert ex[k] is None
    assert np.array_equal(ex["h"], full["h"]) and np.array_equal(ex["mask"], full["mask"])


@pytest.mark.parametrize("p", [0.0, 0.3])
def test_exit_backward_matches_torch_autograd(olib, p):
    d = oracle.Desc(s_local=8, b=2, h=64, io=F32, norm=LN, p=p, seed=3)
    inp = make_inputs(d.rows, d.h, F32, seed=44, dh_out=True)
    out = oracle.fwd(d, inp["x"], inp["bias"], inp["residual"], None, None, L=olib)
    g = oracle.bwd(d, None, inp["dh_out"], None, out["mask"], None, None, None, L=olib)
    assert g["dgamma"] is None and g["dbeta"] is None
    keep = np.ones(d.rows * d.h) if p == 0 else out["mask"].astype(np.float64)
    scale = float(oracle.dropout_scale(p, L=olib)) if p > 0 else 1.0
    x = torch.tensor(inp["x"].astype(np.float64), requires_grad=True)
    b = torch.tensor(inp["bias"].astype(np.float64), requires_grad=True)
    r = torch.tensor(inp["residual"].astype(np.float64), requires_grad=True)
    u = (x.view(d.rows, d.h) + b).view(-1)
    h = r + torch.from_numpy(keep) * scale * u
    (h * torch.from_numpy(inp["dh_out"].astype(np.float64))).sum().backward()
    for k, v in (("dx", x.grad), ("dres", r.grad), ("dbias", b.grad)):
        v = v.numpy()
        rel = np.max(np.abs(g[k].astype(np.float64) - v)) / np.max(np.abs(v))
        assert rel <= 1e-6, (k, rel)
    assert np.array_equal(g["dres"], inp["dh_out"])           # dres is dh_out exactly


def test_variant_argument_rules(olib):
    d = oracle.Desc(s_local=2, b=1, h=8, io=F32, norm=LN, p=0.1)
    inp = make_inputs(d.rows, d.h, F32, seed=45)
    with pytest.raises(ValueError):            # neither branch nor norm
        oracle.fwd(d, None, None, inp["residual"], None, None, L=olib)
    with pytest.raises(ValueError):            # entry with dropout (no branch to drop)
        oracle.fwd(d, None, None, inp["residual"], inp["gamma"], inp["beta"], L=olib)
    d0 = oracle.Desc(s_local=2, b=1, h=8, io=F32, norm=LN, p=0.0)
    with pytest.raises(ValueError):            # entry with a bias
        oracle.fwd(d0, None, inp["bias"], inp["residual"], inp["gamma"], inp["beta"], L=olib)

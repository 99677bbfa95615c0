"""Pins of the oracle's forward and backward.

The forward is pinned by the p = 0 identity, the inverted-dropout
expectation, the LayerNorm / RMSNorm closed forms, and torch's float64
layer_norm / rms_norm; the backward by central finite differences of the
all-float64 forward, by torch float64 autograd, and by the LayerNorm identity
sum_c dh = 0.  Shard invariance follows from per-token independence ("Sequence
parallel math", section "The move: split the LayerNorm/dropout band along the
sequence"; "SP: Partition Activations Alongside TP", section "Normalize and
add residuals by token").
"""
import numpy as np
import pytest
import torch

import oracle
from sp_inputs import make_inputs

F32, BF16, LN, RMS = oracle.F32, oracle.BF16, oracle.LAYERNORM, oracle.RMSNORM


def _widen(d, a):
    return oracle.bf16_to_f32(a) if d.io == BF16 else np.asarray(a, np.float32)


def _run_fwd(olib, d, inp, with_bias=True):
    return oracle.fwd(d, inp["x"], inp["bias"] if with_bias else None, inp["residual"],
                      inp["gamma"], inp["beta"] if d.norm == LN else None, L=olib)


# ------------------------------------------------------------------ forward
@pytest.mark.parametrize("io", [F32, BF16])
def test_p0_is_identity_dropout(olib, io):
    d = oracle.Desc(s_local=16, b=2, h=64, io=io, norm=LN, p=0.0, eps=1e-5)
    inp = make_inputs(d.rows, d.h, io, seed=1)
    out = _run_fwd(olib, d, inp)
    assert out["mask"] is None
    x, r = _widen(d, inp["x"]).reshape(-1, d.h), _widen(d, inp["residual"]).reshape(-1, d.h)
    want = (r + (x + inp["bias"]))                   # fp32 numpy, one rounding per op
    want = oracle.f32_to_bf16(want, L=olib) if io == BF16 else want.ravel()
    assert np.array_equal(out["h"].view(np.uint32 if io == F32 else np.uint16),
                          np.asarray(want).ravel().view(np.uint32 if io == F32 else np.uint16))


def test_dropout_drops_to_residual_and_keeps_expectation(olib):
    # x = c, bias = 0: dropped elements leave h == residual exactly, kept ones
    # add c * scale, and the mean added value is c (inverted dropout).
    p, c = 0.25, np.float32(0.75)
    d = oracle.Desc(s_local=512, b=1, h=256, io=F32, norm=LN, p=p, eps=1e-5, seed=9)
    rng = np.random.default_rng(2)
    res = rng.standard_normal(d.rows * d.h, dtype=np.float32)
    x = np.full(d.rows * d.h, c, np.float32)
    out = oracle.fwd(d, x, None, res, np.ones(d.h, np.float32), np.zeros(d.h, np.float32), L=olib)
    keep = out["mask"].astype(bool)
    added = out["h"].astype(np.float64) - res.astype(np.float64)
    assert np.array_equal(out["h"][~keep], res[~keep])
    scale = 1.0 / (1.0 - p)
    assert np.allclose(added[keep], c * scale, rtol=1e-6, atol=1e-6)
    q = keep.mean()
    n = keep.size
    assert abs(q - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n)
    # E[added] = c: within the binomial spread of the kept count
    assert abs(added.mean() - c) < 5 * c * scale * np.sqrt(p * (1 - p) / n)


@pytest.mark.parametrize("norm", [LN, RMS])
def test_norm_closed_forms_unit_affine(olib, norm):
    d = oracle.Desc(s_local=32, b=2, h=96, io=F32, norm=norm, p=0.1, eps=1e-3, seed=4)
    inp = make_inputs(d.rows, d.h, F32, seed=3)
    g1, b0 = np.ones(d.h), np.zeros(d.h)
    ex = oracle.fwd_exact(d, inp["x"], inp["bias"], inp["residual"], g1,
                          b0 if norm == LN else None, L=olib)
    h = ex["h"].reshape(d.rows, d.h)
    y = ex["y"].reshape(d.rows, d.h)
    if norm == LN:
        var = np.var(h, axis=1)                        # population variance
        assert np.allclose(y.mean(axis=1), 0.0, atol=1e-13)
        assert np.allclose(np.var(y, axis=1), var / (var + d.eps), rtol=1e-12)
        assert np.allclose(ex["mean"], h.mean(axis=1), rtol=1e-13)
    else:
        ms = np.mean(h * h, axis=1)
        assert np.allclose(np.mean(y * y, axis=1), ms / (ms + d.eps), rtol=1e-12)
        assert np.allclose(y / h, (1.0 / np.sqrt(ms + d.eps))[:, None], rtol=1e-12)


def test_constant_row_gives_beta(olib):
    d = oracle.Desc(s_local=4, b=1, h=32, io=F32, norm=LN, p=0.0, eps=1e-5)
    x = np.full(d.rows * d.h, 1.5, np.float32)
    res = np.zeros_like(x)
    beta = np.linspace(-1, 1, d.h).astype(np.float32)
    out = oracle.fwd(d, x, None, res, np.full(d.h, 3.0, np.float32), beta, L=olib)
    assert np.array_equal(out["y"].reshape(d.rows, d.h), np.tile(beta, (d.rows, 1)))


@pytest.mark.parametrize("norm", [LN, RMS])
@pytest.mark.parametrize("io", [F32, BF16])
def test_forward_matches_torch_float64_norm(olib, norm, io):
    d = oracle.Desc(s_local=24, b=3, h=200, io=io, norm=norm, p=0.1, eps=1e-5, seed=2)
    inp = make_inputs(d.rows, d.h, io, seed=5)
    beta = inp["beta"] if norm == LN else None
    out = oracle.fwd(d, inp["x"], inp["bias"], inp["residual"], inp["gamma"], beta, L=olib)
    h64 = torch.from_numpy(_widen(d, out["h"]).astype(np.float64).reshape(d.rows, d.h))
    g64 = torch.from_numpy(inp["gamma"].astype(np.float64))
    if norm == LN:
        ref = torch.nn.functional.layer_norm(h64, (d.h,), g64,
                                             torch.from_numpy(beta.astype(np.float64)), d.eps)
    else:
        ref = torch.nn.functional.rms_norm(h64, (d.h,), g64, d.eps)
    ref32 = ref.numpy().astype(np.float32).ravel()
    got = _widen(d, out["y"])
    if io == F32:
        ulps = np.abs(got.view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
        assert ulps.max() <= 1
    else:
        ref16 = oracle.bf16_to_f32(oracle.f32_to_bf16(ref32, L=olib))
        assert np.all(np.abs(got - ref16) <= np.spacing(np.abs(ref16).astype(np.float32)) * 2**16)
    # the statistics are those of the rounded h
    hh = h64.numpy()
    if norm == LN:
        assert np.allclose(out["mean"], hh.mean(axis=1), rtol=1e-6, atol=1e-7)
        assert np.allclose(out["rstd"], 1 / np.sqrt(hh.var(axis=1) + d.eps), rtol=1e-6)
    else:
        assert np.allclose(out["rstd"], 1 / np.sqrt((hh * hh).mean(axis=1) + d.eps), rtol=1e-6)


@pytest.mark.parametrize("mean", [1.0e4, -2.0e3])
def test_layernorm_is_shift_invariant_on_large_mean_rows(olib, mean):
    """LayerNorm of rows whose mean is 10^3-10^4 times their spread (fp32
    I/O, p = 0): the oracle's y equals torch's float64 layer_norm of the same
    rounded h to one fp32 ulp, and its variance is that of the row with the
    mean subtracted exactly (the statistics do not lose the spread to the
    mean)."""
    d = oracle.Desc(s_local=9, b=2, h=300, io=F32, norm=LN, p=0.0, eps=1e-5, seed=4)
    inp = make_inputs(d.rows, d.h, F32, seed=8)
    inp["residual"] = (np.float32(mean) + inp["residual"]).astype(np.float32)
    out = _run_fwd(olib, d, inp)
    h64 = out["h"].astype(np.float64).reshape(d.rows, d.h)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(h64), (d.h,),
                                         torch.from_numpy(inp["gamma"].astype(np.float64)),
                                         torch.from_numpy(inp["beta"].astype(np.float64)),
                                         d.eps).numpy().astype(np.float32).ravel()
    ulps = np.abs(out["y"].view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    centred = h64 - h64.mean(axis=1, keepdims=True)
    assert np.allclose(out["rstd"], 1 / np.sqrt((centred ** 2).mean(axis=1) + d.eps), rtol=1e-6)


# ----------------------------------------------------------------- backward
def _loss(d, ex, dy, dho):
    val = float(np.dot(dy, ex["y"]))
    if dho is not None:
        val += float(np.dot(dho, ex["h"]))
    return val


@pytest.mark.parametrize("norm", [LN, RMS])
@pytest.mark.parametrize("p", [0.0, 0.1, 0.5])
@pytest.mark.parametrize("t,shard", [(1, 0), (2, 1)])
@pytest.mark.parametrize("with_dh_out", [False, True])
def test_backward_matches_finite_differences(olib, norm, p, t, shard, with_dh_out):
    d = oracle.Desc(s_local=4, b=2, h=8, shard_index=shard, t=t, io=F32, norm=norm, p=p,
                    eps=1e-5, seed=17)
    rng = np.random.default_rng(100 + shard)
    n, H = d.rows * d.h, d.h
    args = {"x": rng.standard_normal(n), "bias": rng.standard_normal(H) * 0.1,
            "residual": rng.standard_normal(n), "gamma": 1 + 0.1 * rng.standard_normal(H),
            "beta": rng.standard_normal(H) * 0.1 if norm == LN else None}
    dy = rng.standard_normal(n)
    dho = rng.standard_normal(n) if with_dh_out else None

    def f(a):
        return _loss(d, oracle.fwd_exact(d, a["x"], a["bias"], a["residual"], a["gamma"],
                                         a["beta"], L=olib), dy, dho)

    ex = oracle.fwd_exact(d, **args, L=olib)
    an = oracle.bwd_exact(d, dy, dho, ex["h"], ex["mask"], ex["mean"], ex["rstd"],
                          args["gamma"], L=olib)
    step = 1e-6
    pairs = [("x", "dx"), ("residual", "dres"), ("gamma", "dgamma"), ("bias", "dbias")]
    if norm == LN:
        pairs.append(("beta", "dbeta"))
    for name, gname in pairs:
        fd = np.empty_like(args[name])
        for i in range(args[name].size):
            a_p = {k: (v.copy() if v is not None else None) for k, v in args.items()}
            a_m = {k: (v.copy() if v is not None else None) for k, v in args.items()}
            a_p[name][i] += step
            a_m[name][i] -= step
            fd[i] = (f(a_p) - f(a_m)) / (2 * step)
        g = an[gname]
        err = np.max(np.abs(fd - g))
        assert err <= 1e-6 * max(1.0, np.max(np.abs(g))), (name, err)


def test_layernorm_dh_sums_to_zero_per_row(olib):
    d = oracle.Desc(s_local=8, b=2, h=64, io=F32, norm=LN, p=0.0, eps=1e-5)
    rng = np.random.default_rng(8)
    n = d.rows * d.h
    ex = oracle.fwd_exact(d, rng.standard_normal(n), None, rng.standard_normal(n),
                          1 + 0.1 * rng.standard_normal(d.h), rng.standard_normal(d.h), L=olib)
    an = oracle.bwd_exact(d, rng.standard_normal(n), None, ex["h"], None, ex["mean"],
                          ex["rstd"], 1 + 0.1 * rng.standard_normal(d.h), L=olib)
    sums = an["dres"].reshape(d.rows, d.h).sum(axis=1)
    assert np.max(np.abs(sums)) < 1e-12 * np.max(np.abs(an["dres"])) * d.h


def _torch_grads(d, x, bias, res, gamma, beta, mask, dy, dho):
    def T(a, shape=None):
        a = np.asarray(a, np.float64)
        return torch.tensor(a if shape is None else a.reshape(shape), requires_grad=True)
    tx, tr = T(x, (d.rows, d.h)), T(res, (d.rows, d.h))
    tb, tg = T(bias), T(gamma)
    leaves = [tx, tb, tr, tg]
    keep = torch.ones(d.rows, d.h, dtype=torch.float64) if mask is None else \
        torch.from_numpy(mask.reshape(d.rows, d.h).astype(np.float64))
    scale = oracle.dropout_scale(d.p)
    h = tr + (tx + tb) * keep * scale
    if d.norm == LN:
        tbeta = T(beta)
        leaves.append(tbeta)
        y = torch.nn.functional.layer_norm(h, (d.h,), tg, tbeta, d.eps)
    else:
        y = torch.nn.functional.rms_norm(h, (d.h,), tg, d.eps)
    loss = (y * torch.from_numpy(np.asarray(dy, np.float64).reshape(d.rows, d.h))).sum()
    if dho is not None:
        loss = loss + (h * torch.from_numpy(np.asarray(dho, np.float64).reshape(d.rows, d.h))).sum()
    loss.backward()
    g = {"dx": tx.grad.numpy().ravel(), "dbias": tb.grad.numpy(), "dres": tr.grad.numpy().ravel(),
         "dgamma": tg.grad.numpy()}
    if d.norm == LN:
        g["dbeta"] = leaves[4].grad.numpy()
    return g


@pytest.mark.parametrize("norm", [LN, RMS])
def test_backward_matches_torch_autograd(olib, norm):
    d = oracle.Desc(s_local=16, b=2, h=128, io=F32, norm=norm, p=0.1, eps=1e-5, seed=21)
    inp = make_inputs(d.rows, d.h, F32, seed=6, dh_out=True)
    beta = inp["beta"] if norm == LN else None
    # all-float64 oracle vs torch float64 autograd
    ex = oracle.fwd_exact(d, inp["x"], inp["bias"], inp["residual"], inp["gamma"], beta, L=olib)
    an = oracle.bwd_exact(d, inp["dy"], inp["dh_out"], ex["h"], ex["mask"], ex["mean"],
                          ex["rstd"], inp["gamma"], L=olib)
    ref = _torch_grads(d, inp["x"], inp["bias"], inp["residual"], inp["gamma"], beta,
                       ex["mask"], inp["dy"], inp["dh_out"])
    for k, v in ref.items():
        assert np.max(np.abs(an[k] - v)) <= 1e-10 * max(1.0, np.max(np.abs(v))), k
    # production (fp32 I/O, fp32 stored stats) vs the same reference
    out = oracle.fwd(d, inp["x"], inp["bias"], inp["residual"], inp["gamma"], beta, L=olib)
    assert np.array_equal(out["mask"], ex["mask"])
    gb = oracle.bwd(d, inp["dy"], inp["dh_out"], out["h"], out["mask"], out["mean"], out["rstd"],
                    inp["gamma"], L=olib)
    for k, v in ref.items():
        rel = np.max(np.abs(gb[k].astype(np.float64) - v)) / np.max(np.abs(v))
        assert rel <= 1e-5, (k, rel)


# --------------------------------------------------------- shard invariance
@pytest.mark.parametrize("io,norm", [(F32, LN), (BF16, LN), (BF16, RMS)])
@pytest.mark.parametrize("t", [2, 4])
def test_shards_concatenate_to_unsharded_run(olib, io, norm, t):
    s, b, H = 16, 2, 64
    full = oracle.Desc(s_local=s, b=b, h=H, shard_index=0, t=1, io=io, norm=norm, p=0.1,
                       eps=1e-5, seed=31, offset=2)
    inp = make_inputs(full.rows, H, io, seed=12, dh_out=True)
    beta = inp["beta"] if norm == LN else None
    ref = oracle.fwd(full, inp["x"], inp["bias"], inp["residual"], inp["gamma"], beta, L=olib)
    refb = oracle.bwd(full, inp["dy"], inp["dh_out"], ref["h"], ref["mask"], ref["mean"],
                      ref["rstd"], inp["gamma"], L=olib)
    N = full.rows // t
    acc = {k: np.zeros(H, np.float64) for k in ("dgamma", "dbeta", "dbias") if refb[k] is not None}
    for i in range(t):
        d = oracle.Desc(s_local=s // t, b=b, h=H, shard_index=i, t=t, io=io, norm=norm, p=0.1,
                        eps=1e-5, seed=31, offset=2)
        sl = slice(i * N * H, (i + 1) * N * H)
        o = oracle.fwd(d, inp["x"][sl], inp["bias"], inp["residual"][sl], inp["gamma"], beta,
                       L=olib)
        for k in ("h", "y", "mask"):
            assert np.array_equal(o[k], ref[k][sl]), k
        for k in ("mean", "rstd"):
            if o[k] is not None:
                assert np.array_equal(o[k], ref[k][i * N:(i + 1) * N]), k
        g = oracle.bwd(d, inp["dy"][sl], inp["dh_out"][sl], o["h"], o["mask"], o["mean"],
                       o["rstd"], inp["gamma"], L=olib)
        for k in ("dx", "dres"):
            assert np.array_equal(g[k], refb[k][sl]), k
        for k in acc:
            acc[k] += g[k]
    for k in acc:
        rel = np.max(np.abs(acc[k] - refb[k])) / np.max(np.abs(refb[k]))
        assert rel <= 1e-5, k


def test_two_gpu_toy_layout(olib):
    # "SP: Partition Activations Alongside TP", section "Normalize and add
    # residuals by token": 4 tokens x 4 features on 2 GPUs; GPU 0 holds t0, t1
    # and GPU 1 holds t2, t3, whole token vectors.  Each shard's output is the
    # matching half of the unsharded result.
    full = oracle.Desc(s_local=4, b=1, h=4, t=1, io=F32, norm=RMS, p=0.5, eps=1e-6, seed=1)
    inp = make_inputs(4, 4, F32, seed=0)
    ref = oracle.fwd(full, inp["x"], None, inp["residual"], inp["gamma"], None, L=olib)
    for gpu in (0, 1):
        d = oracle.Desc(s_local=2, b=1, h=4, shard_index=gpu, t=2, io=F32, norm=RMS, p=0.5,
                        eps=1e-6, seed=1)
        sl = slice(gpu * 8, gpu * 8 + 8)
        o = oracle.fwd(d, inp["x"][sl], None, inp["residual"][sl], inp["gamma"], None, L=olib)
        assert np.array_equal(o["y"], ref["y"][sl]) and np.array_equal(o["mask"], ref["mask"][sl])


def test_row_range_calls_match_whole_shard(olib):
    d = oracle.Desc(s_local=8, b=2, h=48, shard_index=1, t=3, io=BF16, norm=LN, p=0.1,
                    eps=1e-5, seed=5)
    inp = make_inputs(d.rows, d.h, BF16, seed=9)
    whole = oracle.fwd(d, inp["x"], inp["bias"], inp["residual"], inp["gamma"], inp["beta"],
                       L=olib)
    r0, r1 = 5, 11
    sl = slice(r0 * d.h, r1 * d.h)
    part = oracle.fwd(d, inp["x"][sl], inp["bias"], inp["residual"][sl], inp["gamma"],
                      inp["beta"], rows=(r0, r1), L=olib)
    for k in ("h", "y", "mask"):
        assert np.array_equal(part[k], whole[k][sl])
    assert np.array_equal(part["rstd"], whole["rstd"][r0:r1])


def test_invalid_arguments_are_rejected(olib):
    inp = make_inputs(4, 8, F32, seed=0)
    base = dict(s_local=4, b=1, h=8, io=F32, norm=LN, p=0.1, eps=1e-5)
    bad = [dict(base, p=1.0), dict(base, p=-0.1), dict(base, eps=0.0), dict(base, t=0),
           dict(base, shard_index=1, t=1), dict(base, h=0), dict(base, io=7), dict(base, norm=3)]
    for kw in bad:
        with pytest.raises(ValueError):
            oracle.fwd(oracle.Desc(**kw), inp["x"], None, inp["residual"], inp["gamma"],
                       inp["beta"], L=olib)
    with pytest.raises(ValueError):      # beta given for RMSNorm
        oracle.fwd(oracle.Desc(**dict(base, norm=RMS)), inp["x"], None, inp["residual"],
                   inp["gamma"], inp["beta"], L=olib)

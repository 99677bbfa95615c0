"""GPU parity on rows the usual draws never produce.

* Constant rows (every h of the row equal): the variance is 0, so
  rstd = 1/sqrt(eps) and y = beta (LayerNorm) or sign(h) * gamma / sqrt(1 +
  eps/h^2) (RMSNorm); the backward sees xhat = 0 and a large rstd.
* fp32 rows whose mean is 10^3-10^4 times their spread: a one-pass variance
  (E[h^2] - E[h]^2 in fp32) would lose every digit here.  The statistics
  must meet the 1e-5 relative tolerance and y the fp32 1e-5 max-abs one,
  like any other row: the kernel subtracts a pivot taken from the row before
  it forms any sum, so no fp32 number of the size of the mean ever enters
  the normalised value ((h - pivot) - mean_rel) * rstd.  The backward on the
  same rows (both paths) must meet the usual gradient tolerances.
"""
import zlib

import numpy as np
import pytest

import dropout_region_amd as spr
import oracle
from sp_inputs import make_inputs, to_bf16_bits
from tests import parity as P

pytestmark = pytest.mark.gpu

F32, BF16, LN, RMS = spr.SPR_F32, spr.SPR_BF16, spr.SPR_LAYERNORM, spr.SPR_RMSNORM


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    spr.lib()


def _descs(**kw):
    return spr.Desc(**kw), oracle.Desc(**kw)


CONST = {
    "bf16_ln_h6144": dict(s_local=5, b=2, h=6144, io=BF16, norm=LN),
    "bf16_rms_h8192": dict(s_local=5, b=1, h=8192, io=BF16, norm=RMS, eps=1e-6),
    "fp32_ln_h256_wave_rows": dict(s_local=5, b=2, h=256, io=F32, norm=LN),
    "bf16_ln_h25600_split": dict(s_local=5, b=1, h=25600, io=BF16, norm=LN),
}
ROW_VALUES = np.array([0.5, -3.0, 0.0, 1024.0, 1.0 / 3.0], np.float32)


@pytest.mark.parametrize("name", sorted(CONST))
def test_constant_rows(name):
    kw = dict(shard_index=0, t=1, p=0.0, eps=1e-5, seed=0, offset=0)
    kw.update(CONST[name])
    d, od = _descs(**kw)
    _say(f"[case] constant rows {name}: {kw}")
    inp = make_inputs(d.rows, d.h, d.io, seed=zlib.crc32(name.encode()) % 1000)
    vals = np.resize(ROW_VALUES, d.rows)
    res = np.repeat(vals, d.h).astype(np.float32)
    cast = to_bf16_bits if d.io == BF16 else (lambda a: a)
    inp["residual"] = cast(res)
    inp["x"] = cast(np.zeros(d.rows * d.h, np.float32))      # h = residual + 0 exactly
    want = P.oracle_fwd(od, inp, with_bias=False)
    for path in (None, "rows", "stream"):
        got = P.gpu_fwd(d, inp, with_bias=False, path=path)
        P.check_fwd(got, want, d.io)
    wb = P.oracle_bwd(od, inp, want, want_dbias=True)
    gb = P.gpu_bwd(d, inp, want, want_dbias=True, repeat=2)
    P.check_bwd(gb, wb, d.io)
    for path in ("fused", "split"):
        gb = P.gpu_bwd(d, inp, want, want_dbias=True, path=path)
        P.check_bwd(gb, wb, d.io)


@pytest.mark.parametrize("h,mean", [(256, 1.0e4), (6144, 1.0e4), (3076, -2.0e3)])
def test_large_mean_rows_fp32(h, mean):
    kw = dict(s_local=7, b=3, h=h, shard_index=1, t=2, io=F32, norm=LN, p=0.1, eps=1e-5,
              seed=3, offset=1)
    d, od = _descs(**kw)
    _say(f"[case] large-mean rows: {kw}, mean {mean}")
    inp = make_inputs(d.rows, d.h, d.io, seed=h)
    inp["residual"] = (np.float32(mean) + inp["residual"]).astype(np.float32)
    inp["x"] = (np.float32(0.1) * inp["x"]).astype(np.float32)
    want = P.oracle_fwd(od, inp)
    for path in (None, "rows", "stream"):
        got = P.gpu_fwd(d, inp, path=path)
        _say(f"[case] large-mean rows, forward kernel {path or 'auto'}")
        P.check_fwd(got, want, d.io)
    wb = P.oracle_bwd(od, inp, want, want_dbias=True)
    for path in ("fused", "split"):
        _say(f"[case] large-mean rows, backward path {path}")
        gb = P.gpu_bwd(d, inp, want, want_dbias=True, repeat=2, path=path)
        P.check_bwd(gb, wb, d.io)

"""The ring-attention comparison rule (tests/attn_check.py) on the CPU.

An emulation of the kernel's rounding -- the probabilities rounded to bf16
before P V, the row sum of the unrounded ones, O rounded to bf16 once --
must pass the rule; the same emulation with a key-local mistake of the kind
a transposed-V staging bug makes (two keys of every 64-key tile read each
other's values), or with one key of every tile dropped, must fail it.  The
emulation is numpy float32 arithmetic written here, not the kernel and not
the oracle."""
import numpy as np
import pytest

import oracle
from sp_inputs import make_attn_inputs, make_attn_inputs_matched, to_bf16_bits
from tests.attn_check import check_attention


def _f(bits):
    return oracle.bf16_to_f32(bits)


def _bf16(a):
    return _f(to_bf16_bits(np.asarray(a, np.float32)))


def emulate(od, x, mistake=None):
    """O (bf16 bits) and lse of the kernel's arithmetic in numpy float32."""
    S, T, D = od.s_local, od.t * od.s_local, od.d
    bh = od.b * od.heads
    scale = np.float32(1.0 / np.sqrt(D))
    q = _f(x["q"]).reshape(S, bh, D).transpose(1, 0, 2)
    k = _f(x["k"]).reshape(T, bh, D).transpose(1, 2, 0)
    v = _f(x["v"]).reshape(T, bh, D).transpose(1, 0, 2).copy()
    s = np.matmul(q, k) * scale                                   # float32 [bh, S, T]
    p = np.exp(s - s.max(axis=2, keepdims=True)).astype(np.float32)
    l = p.sum(axis=2, dtype=np.float32)
    pb = _bf16(p)
    if mistake == "swap":                  # keys 5 and 9 of every tile trade values
        idx = np.arange(T)
        for t0 in range(0, T - 9, 64):
            idx[t0 + 5], idx[t0 + 9] = t0 + 9, t0 + 5
        v = v[:, idx, :]
    elif mistake == "drop":                # key 17 of every tile is left out
        for t0 in range(0, T - 17, 64):
            pb[:, :, t0 + 17] = 0.0
    o = np.matmul(pb, v) / l[:, :, None]
    lse = np.log(l.astype(np.float64)) + s.max(axis=2)
    o = o.transpose(1, 0, 2).reshape(-1)
    return to_bf16_bits(o.astype(np.float32)), lse.T.reshape(-1).astype(np.float32)


CASES = {
    "random_d128_t4": (dict(s_local=96, b=1, heads=2, d=128, t=4, rank=1), False),
    "random_d64_t8": (dict(s_local=64, b=1, heads=2, d=64, t=8, rank=3), False),
    "matched_d128_t4": (dict(s_local=96, b=1, heads=1, d=128, t=4, rank=1), True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_rule_accepts_the_kernels_rounding_and_rejects_layout_mistakes(name, olib):
    kw, matched = CASES[name]
    od = oracle.AttnDesc(**kw)
    gen = make_attn_inputs_matched if matched else make_attn_inputs
    x = gen(od.s_local, od.b, od.heads, od.d, od.t, seed=5)
    want_o, want_lse = oracle.attention(od, x["q"], x["k"], x["v"])
    o, lse = emulate(od, x)
    check_attention(name, od, x["q"], x["k"], x["v"], o, lse, want_o, want_lse)
    for mistake in ("swap", "drop"):
        o_bad, _ = emulate(od, x, mistake)
        with pytest.raises(AssertionError):
            check_attention(f"{name} {mistake}", od, x["q"], x["k"], x["v"], o_bad, None,
                            want_o, want_lse)

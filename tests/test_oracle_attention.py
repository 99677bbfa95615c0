"""Pins of the oracle's ring attention (spo_attention): ordinary attention of
one rank's queries over the keys of all t blocks, in float64.

Pinned against torch's float64 scaled_dot_product_attention, closed forms
(a single key, identical keys, constant values, two keys), and the
invariance of the result to the order of the key blocks (the ring order)."""
import numpy as np
import pytest
import torch

import oracle
from sp_inputs import make_attn_inputs, to_bf16_bits


def _w(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def _scale(dim):
    """The softmax scale as the descriptor carries it: fp32(1/sqrt(d))."""
    return float(np.float32(1.0 / np.sqrt(dim)))


def _bshd(a, tokens, d):
    return a.reshape(tokens, d.b, d.heads, d.d)


@pytest.mark.parametrize("s_local,b,heads,dim,t,rank", [(5, 2, 3, 16, 3, 1), (8, 1, 2, 32, 4, 3),
                                                        (3, 3, 1, 8, 1, 0)])
def test_matches_torch_sdpa_float64(olib, s_local, b, heads, dim, t, rank):
    d = oracle.AttnDesc(s_local=s_local, b=b, heads=heads, d=dim, t=t, rank=rank)
    x = make_attn_inputs(s_local, b, heads, dim, t, seed=7)
    o, lse = oracle.attention(d, x["q"], x["k"], x["v"], L=olib)
    # torch wants [batch, heads, tokens, d]
    q = torch.from_numpy(_bshd(_w(x["q"]), s_local, d)).permute(1, 2, 0, 3)
    k = torch.from_numpy(_bshd(_w(x["k"]), t * s_local, d)).permute(1, 2, 0, 3)
    v = torch.from_numpy(_bshd(_w(x["v"]), t * s_local, d)).permute(1, 2, 0, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=_scale(dim))
    ref = ref.permute(2, 0, 1, 3).numpy().ravel()
    assert np.max(np.abs(o - ref)) <= 1e-12
    scores = torch.einsum("bhqd,bhkd->bhqk", q, k) * _scale(dim)
    ref_lse = torch.logsumexp(scores, dim=-1).permute(2, 0, 1).numpy().ravel()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_single_key_returns_its_value(olib):
    d = oracle.AttnDesc(s_local=1, b=1, heads=2, d=8, t=1)
    x = make_attn_inputs(1, 1, 2, 8, 1, seed=3)
    o, lse = oracle.attention(d, x["q"], x["k"], x["v"], L=olib)
    assert np.array_equal(o, _w(x["v"]))
    q, k = _w(x["q"]).reshape(2, 8), _w(x["k"]).reshape(2, 8)
    assert np.allclose(lse, (q * k).sum(axis=1) * _scale(8), rtol=0, atol=1e-15)


def test_identical_keys_average_the_values(olib):
    s_local, t, dim = 4, 3, 16
    d = oracle.AttnDesc(s_local=s_local, b=1, heads=1, d=dim, t=t)
    x = make_attn_inputs(s_local, 1, 1, dim, t, seed=4)
    k = np.tile(x["k"][:dim], t * s_local)               # every key the same
    o, lse = oracle.attention(d, x["q"], k, x["v"], L=olib)
    mean_v = _w(x["v"]).reshape(t * s_local, dim).mean(axis=0)
    assert np.allclose(o.reshape(s_local, dim), mean_v, rtol=0, atol=1e-14)
    q = _w(x["q"]).reshape(s_local, dim)
    s = q @ _w(k[:dim]) * _scale(dim)
    assert np.allclose(lse, s + np.log(t * s_local), rtol=0, atol=1e-13)


def test_constant_values_pass_through(olib):
    d = oracle.AttnDesc(s_local=6, b=2, heads=2, d=8, t=2)
    x = make_attn_inputs(6, 2, 2, 8, 2, seed=5)
    v = np.tile(to_bf16_bits(np.linspace(-2, 2, 8, dtype=np.float32)), 2 * 6 * 2 * 2)
    o, _ = oracle.attention(d, x["q"], x["k"], v, L=olib)
    assert np.allclose(o.reshape(-1, 8), _w(v[:8]), rtol=0, atol=1e-14)


def test_two_keys_closed_form(olib):
    d = oracle.AttnDesc(s_local=1, b=1, heads=1, d=4, t=2, scale=0.5)
    q = to_bf16_bits(np.array([1, 0, 0, 0], np.float32))
    k = to_bf16_bits(np.array([2, 0, 0, 0, -1, 0, 0, 0], np.float32))
    v = to_bf16_bits(np.array([1, 2, 3, 4, -4, -3, -2, -1], np.float32))
    o, lse = oracle.attention(d, q, k, v, L=olib)
    w1, w2 = np.exp(0.5 * 2), np.exp(0.5 * -1)
    want = (w1 * np.array([1, 2, 3, 4]) + w2 * np.array([-4, -3, -2, -1])) / (w1 + w2)
    assert np.allclose(o, want, rtol=0, atol=1e-15)
    assert abs(lse[0] - np.log(w1 + w2)) <= 1e-15


def test_result_does_not_depend_on_the_ring_order(olib):
    s_local, b, heads, dim, t = 4, 2, 2, 16, 4
    x = make_attn_inputs(s_local, b, heads, dim, t, seed=6)
    blk = s_local * b * heads * dim
    ref = None
    for rank in range(t):
        d = oracle.AttnDesc(s_local=s_local, b=b, heads=heads, d=dim, t=t, rank=rank)
        order = [(rank - k) % t for k in range(t)]       # the blocks in ring order
        k = np.concatenate([x["k"][j * blk:(j + 1) * blk] for j in order])
        v = np.concatenate([x["v"][j * blk:(j + 1) * blk] for j in order])
        o, lse = oracle.attention(d, x["q"], k, v, L=olib)
        if ref is None:
            ref = (o, lse)
        assert np.allclose(o, ref[0], rtol=0, atol=1e-13)
        assert np.allclose(lse, ref[1], rtol=0, atol=1e-13)


def test_query_ranges_concatenate(olib):
    s_local, b, heads, dim, t = 6, 2, 2, 16, 2
    d = oracle.AttnDesc(s_local=s_local, b=b, heads=heads, d=dim, t=t)
    x = make_attn_inputs(s_local, b, heads, dim, t, seed=8)
    o, lse = oracle.attention(d, x["q"], x["k"], x["v"], L=olib)
    tok = b * heads * dim
    for r0, r1 in ((0, 2), (2, 5), (5, 6)):
        oo, ll = oracle.attention(d, x["q"][r0 * tok:r1 * tok], x["k"], x["v"], rows=(r0, r1),
                                  L=olib)
        assert np.array_equal(oo, o[r0 * tok:r1 * tok])
        assert np.array_equal(ll, lse[r0 * b * heads:r1 * b * heads])


def test_rejects_bad_arguments(olib):
    x = make_attn_inputs(2, 1, 1, 8, 2, seed=1)
    with pytest.raises(ValueError):
        oracle.attention(oracle.AttnDesc(s_local=2, b=1, heads=1, d=8, t=2, rank=2),
                         x["q"], x["k"], x["v"], L=olib)

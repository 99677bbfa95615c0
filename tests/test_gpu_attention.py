"""GPU parity of the ring-attention forward (include/sp_ring_attn.h) against
the oracle's ordinary attention over all keys.  The comparison rule, derived
from the kernel's arithmetic, is tests/attn_check.py: per element
|O_gpu - O| <= ulp_bf16(O) + (2^-8 + 2^-12 + score term) * sum_j w_j |v_j|,
the mean square error within 4 times its expectation from the bf16 rounding
of the probabilities, and lse within 1e-4 + 1e-5 |lse|."""
import zlib

import numpy as np
import pytest

import dropout_region_amd as spr
import oracle
from sp_inputs import make_attn_inputs, make_attn_inputs_matched, make_attn_inputs_ramp
from tests.attn_check import check_attention as _check
from tests import parity as P

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    spr.lib()


def _dev(bits):
    return P.to_device(bits, P.BF16)


def _spg(d, k):
    """d with k ring steps per workgroup (0: the library's choice)."""
    import dataclasses
    return dataclasses.replace(d, steps_per_wg=k)


def check_attention(name, od, x, got_o, got_lse, want_o, want_lse, rows=None):
    """x: the inputs (bf16 bits); q is the whole rank's queries unless rows
    names a range of them."""
    q = x["q"]
    if rows is not None:
        tok = od.b * od.heads * od.d
        q = q[rows[0] * tok:rows[1] * tok]
    _check(name, od, q, x["k"], x["v"], got_o, got_lse, want_o, want_lse, rows=rows)


CASES = {
    "d128_t6_two_ragged_blocks": dict(s_local=70, b=1, heads=2, d=128, t=6, rank=4),
    "d64_one_token_t8_rank3": dict(s_local=1, b=2, heads=3, d=64, t=8, rank=3),
    "d128_full_tiles_t4_rank1": dict(s_local=256, b=1, heads=2, d=128, t=4, rank=1),
    "d64_ragged_b2_t3_rank2": dict(s_local=100, b=2, heads=3, d=64, t=3, rank=2),
    "d128_one_token_t1": dict(s_local=1, b=1, heads=1, d=128, t=1, rank=0),
    "d64_two_tiles_ragged_t2": dict(s_local=130, b=1, heads=4, d=64, t=2, rank=0),
    "d128_t8_rank7": dict(s_local=64, b=1, heads=2, d=128, t=8, rank=7),
    "d128_given_scale": dict(s_local=70, b=2, heads=1, d=128, t=2, rank=1, scale=0.05),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_ring_attention_matches_oracle(name):
    """Every case with the workgroups taking one ring step each, all t steps
    each (one run of key tiles across the blocks, one partial), and the
    launch's own choice."""
    kw = CASES[name]
    d, od = spr.AttnDesc(**kw), oracle.AttnDesc(**kw)
    x = make_attn_inputs(d.s_local, d.b, d.heads, d.d, d.t, seed=zlib.crc32(name.encode()) % 1000)
    want_o, want_lse = oracle.attention(od, x["q"], x["k"], x["v"])
    mid = [k for k in range(2, d.t) if d.t % k == 0][:1]        # a proper divisor, if any
    for spg in sorted({0, 1, d.t, *mid}):
        _say(f"[case] ring attention {name}: {kw}, steps per workgroup {spg or 'auto'}")
        o, lse = spr.ring_attn(_spg(d, spg), _dev(x["q"]), _dev(x["k"]), _dev(x["v"]))
        check_attention(f"{name} spg {spg}", od, x, P.to_host(o), P.to_host(lse), want_o,
                        want_lse)


# Seeded random shapes: any s_local up to 300 (ragged key tiles, ragged
# query tiles), batch and heads up to 3, either head size, any ring size up
# to 8 and any rank, with the launch's own grouping of ring steps.
def _random_attn_cases(n=12, seed=7):
    rng = np.random.default_rng(seed)
    cases = {}
    while len(cases) < n:
        t = int(rng.integers(1, 9))
        kw = dict(s_local=int(rng.integers(1, 301)), b=int(rng.integers(1, 3)),
                  heads=int(rng.integers(1, 4)), d=int(rng.choice([64, 128])), t=t,
                  rank=int(rng.integers(0, t)))
        cases["s{s_local}_b{b}_h{heads}_d{d}_t{t}_r{rank}".format(**kw)] = kw
    return cases


RANDOM_ATTN = _random_attn_cases()


@pytest.mark.parametrize("name", sorted(RANDOM_ATTN))
def test_random_attention_shapes(name):
    kw = RANDOM_ATTN[name]
    d, od = spr.AttnDesc(**kw), oracle.AttnDesc(**kw)
    _say(f"[case] ring attention, random shape {name}")
    x = make_attn_inputs(d.s_local, d.b, d.heads, d.d, d.t, seed=zlib.crc32(name.encode()) % 1000)
    want_o, want_lse = oracle.attention(od, x["q"], x["k"], x["v"])
    o, lse = spr.ring_attn(d, _dev(x["q"]), _dev(x["k"]), _dev(x["v"]))
    check_attention(name, od, x, P.to_host(o), P.to_host(lse), want_o, want_lse)


# Scores that climb along the key sequence by ~200 (base 2) make the streaming
# softmax move its reference (and rescale O) many times, within a tile run,
# across ring-step blocks and in the ring's non-monotone block order; falling
# scores leave the first tile's reference in place.
RAMP = {
    "d64_rising_t4_rank1": (dict(s_local=150, b=1, heads=2, d=64, t=4, rank=1), True),
    "d128_falling_t3_rank2": (dict(s_local=200, b=2, heads=1, d=128, t=3, rank=2), False),
    "d128_rising_t8_rank5": (dict(s_local=70, b=1, heads=1, d=128, t=8, rank=5), True),
}


@pytest.mark.parametrize("name", sorted(RAMP))
def test_softmax_reference_moves(name):
    kw, rising = RAMP[name]
    d, od = spr.AttnDesc(**kw), oracle.AttnDesc(**kw)
    x = make_attn_inputs_ramp(d.s_local, d.b, d.heads, d.d, d.t,
                              seed=zlib.crc32(name.encode()) % 1000, rising=rising)
    want_o, want_lse = oracle.attention(od, x["q"], x["k"], x["v"])
    for spg in sorted({0, 1, d.t}):
        _say(f"[case] ring attention, moving reference {name}: {kw}, steps per workgroup {spg or 'auto'}")
        o, lse = spr.ring_attn(_spg(d, spg), _dev(x["q"]), _dev(x["k"]), _dev(x["v"]))
        check_attention(f"{name} spg {spg}", od, x, P.to_host(o), P.to_host(lse), want_o,
                        want_lse)


MATCHED = {
    "d128_t4_rank1": dict(s_local=150, b=1, heads=2, d=128, t=4, rank=1),
    "d64_t8_rank6_b2": dict(s_local=70, b=2, heads=1, d=64, t=8, rank=6),
    "d128_t2_full_tiles": dict(s_local=256, b=1, heads=1, d=128, t=2, rank=0),
}


@pytest.mark.parametrize("name", sorted(MATCHED))
def test_matched_keys(name):
    """Every query has one key of its own that dominates its softmax, at a
    random position among all the ring's keys: the output is that key's
    value, so a value staged at the wrong key position (the transposed V
    tile's swizzles, the ragged-tile clamp, the ring order) is off by O(1),
    far outside the bound."""
    kw = MATCHED[name]
    d, od = spr.AttnDesc(**kw), oracle.AttnDesc(**kw)
    x = make_attn_inputs_matched(d.s_local, d.b, d.heads, d.d, d.t,
                                 seed=zlib.crc32(name.encode()) % 1000)
    want_o, want_lse = oracle.attention(od, x["q"], x["k"], x["v"])
    # the construction: O is the matched key's value
    v = oracle.bf16_to_f32(x["v"]).reshape(d.t * d.s_local, -1)[x["perm"]].reshape(-1)
    assert np.max(np.abs(want_o - v)) < 1e-4
    for spg in sorted({0, 1, d.t}):
        _say(f"[case] ring attention, matched keys {name}: {kw}, steps per workgroup {spg or 'auto'}")
        o, lse = spr.ring_attn(_spg(d, spg), _dev(x["q"]), _dev(x["k"]), _dev(x["v"]))
        check_attention(f"{name} spg {spg}", od, x, P.to_host(o), P.to_host(lse), want_o,
                        want_lse)


def test_steps_in_any_order_then_merge_equal_the_fused_call():
    import torch
    kw = dict(s_local=192, b=1, heads=3, d=128, t=4, rank=2)
    d = spr.AttnDesc(**kw)
    _say(f"[case] ring attention steps: {kw}")
    x = make_attn_inputs(d.s_local, d.b, d.heads, d.d, d.t, seed=9)
    q, k, v = _dev(x["q"]), _dev(x["k"]), _dev(x["v"])
    o_f, lse_f = spr.ring_attn(_spg(d, 1), q, k, v)   # the fused call, one step per workgroup
    n = d.rows * d.d
    ws = torch.zeros(spr.sp_ring_attn_workspace_bytes(d), dtype=torch.uint8, device=q.device)
    for step in (3, 0, 2, 1):                      # any order: each step has its own slot
        blk = (d.rank - step) % d.t
        spr.sp_ring_attn_step(d, step, q, k[blk * n:(blk + 1) * n], v[blk * n:(blk + 1) * n], ws)
    o = torch.empty_like(o_f)
    spr.sp_ring_attn_merge(d, o, None, ws)        # lse may be omitted
    torch.cuda.synchronize()
    P.exact("o (steps + merge vs fused)", P.to_host(o), P.to_host(o_f))


@pytest.mark.parametrize("spg", [0, 2, 4])
def test_launch_by_launch_equals_the_fused_call(spg):
    """Launching the fused forward's two kernels one at a time on the stream
    (the ring steps, then the merge) gives the bits of sp_ring_attn_fwd."""
    import torch
    kw = dict(s_local=160, b=2, heads=2, d=128, t=4, rank=3)
    d = _spg(spr.AttnDesc(**kw), spg)
    _say(f"[case] ring attention launch by launch: {kw} steps per workgroup {spg or 'auto'}")
    x = make_attn_inputs(d.s_local, d.b, d.heads, d.d, d.t, seed=12)
    q, k, v = _dev(x["q"]), _dev(x["k"]), _dev(x["v"])
    assert spr.sp_ring_attn_fwd_num_launches(d) == 2
    o_f, lse_f = spr.ring_attn(d, q, k, v)
    o = torch.empty_like(o_f)
    lse = torch.empty_like(lse_f)
    ws = torch.zeros(spr.sp_ring_attn_workspace_bytes(d), dtype=torch.uint8, device=q.device)
    for i in range(2):
        spr.sp_ring_attn_fwd_launch(d, i, q, k, v, o, lse, ws)
    torch.cuda.synchronize()
    P.exact("o (launch by launch vs fused)", P.to_host(o), P.to_host(o_f))
    P.exact("lse (launch by launch vs fused)", P.to_host(lse), P.to_host(lse_f))


def test_rank_changes_only_the_order():
    """Every rank of the ring sees the same keys in a different order: the
    results agree within the tolerance (and each matches the oracle)."""
    kw = dict(s_local=128, b=1, heads=2, d=64, t=4)
    x = make_attn_inputs(kw["s_local"], 1, 2, 64, 4, seed=10)
    want_o, want_lse = oracle.attention(oracle.AttnDesc(**kw), x["q"], x["k"], x["v"])
    for rank in range(4):
        d = spr.AttnDesc(rank=rank, **kw)
        o, lse = spr.ring_attn(d, _dev(x["q"]), _dev(x["k"]), _dev(x["v"]))
        check_attention(f"rank {rank}", oracle.AttnDesc(rank=rank, **kw), x, P.to_host(o),
                        P.to_host(lse), want_o, want_lse)


@pytest.mark.parametrize("name", ["ring_attn_s32k_t8_h8192", "ring_attn_s2k_t8_d128"])
def test_full_size_workload_sampled(name):
    """The benchmark's workloads at their real shapes, in the launch the
    benchmark times (every ring step in one call, then the merge); the oracle
    computes a sample of query tokens -- first, last, and a few between --
    over all keys and every (batch, head) pair."""
    from sp_inputs import ATTN_WORKLOADS
    w = ATTN_WORKLOADS[name]
    kw = dict(s_local=w.s_local, b=w.b, heads=w.heads, d=w.d, t=w.t, rank=0)
    _say(f"[case] ring attention full size {name}: {kw}")
    x = make_attn_inputs(w.s_local, w.b, w.heads, w.d, w.t, seed=w.seed)
    o, lse = spr.ring_attn(spr.AttnDesc(**kw), _dev(x["q"]), _dev(x["k"]), _dev(x["v"]))
    go, gl = P.to_host(o), P.to_host(lse)
    od = oracle.AttnDesc(**kw)
    tok, nbh = w.b * w.heads * w.d, w.b * w.heads
    for r in sorted({0, 1, w.s_local // 3, w.s_local // 2 + 7, w.s_local - 2, w.s_local - 1}):
        want_o, want_lse = oracle.attention(od, x["q"][r * tok:(r + 1) * tok], x["k"], x["v"],
                                            rows=(r, r + 1))
        check_attention(f"{name} query {r}", od, x, go[r * tok:(r + 1) * tok],
                        gl[r * nbh:(r + 1) * nbh], want_o, want_lse, rows=(r, r + 1))


def test_graph_replays_and_concurrent_streams_equal_eager():
    """The fused forward captured in a HIP graph and replayed (with eager
    calls between the replays), and two calls of different shapes on two
    streams at once, give the eager bits."""
    import torch
    cases = [spr.AttnDesc(s_local=300, b=1, heads=2, d=128, t=4, rank=1),
             spr.AttnDesc(s_local=130, b=2, heads=1, d=64, t=3, rank=2)]
    print("[case] ring attention: graph replays and two streams", flush=True)
    runs = []
    for i, d in enumerate(cases):
        x = make_attn_inputs(d.s_local, d.b, d.heads, d.d, d.t, seed=30 + i)
        q, k, v = _dev(x["q"]), _dev(x["k"]), _dev(x["v"])
        o_e, lse_e = spr.ring_attn(d, q, k, v)
        torch.cuda.synchronize()
        want = (P.to_host(o_e), P.to_host(lse_e))
        o, lse = torch.empty_like(o_e), torch.empty_like(lse_e)
        ws = torch.zeros(spr.sp_ring_attn_workspace_bytes(d), dtype=torch.uint8, device=q.device)
        runs.append((d, q, k, v, o, lse, ws, want))
    d, q, k, v, o, lse, ws, want = runs[0]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        spr.sp_ring_attn_fwd(d, q, k, v, o, lse, ws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        o.zero_()
        lse.zero_()
        spr.ring_attn(d, q, k, v)                   # eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        P.exact(f"o (replay {rep})", P.to_host(o), want[0])
        P.exact(f"lse (replay {rep})", P.to_host(lse), want[1])
    del g
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(10):
        for (d, q, k, v, o, lse, ws, _), s in zip(runs, streams):
            with torch.cuda.stream(s):
                spr.sp_ring_attn_fwd(d, q, k, v, o, lse, ws)
    torch.cuda.synchronize()
    for d, q, k, v, o, lse, ws, want in runs:
        P.exact(f"o (two streams, s_local {d.s_local})", P.to_host(o), want[0])
        P.exact(f"lse (two streams, s_local {d.s_local})", P.to_host(lse), want[1])

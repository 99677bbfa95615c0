"""Pins of the oracle's dropout generator, threshold, scale and bf16 rounding.

Each check compares the oracle with something other than itself: PyTorch's
header-only Philox4x32-10 engine, torch's float32 -> bfloat16 conversion,
exact rational arithmetic, and binomial / chi-square statistics.
"""
import os
import random
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def build_torch_philox(outdir):
    """Compiles tests/philox_torch_ref.cpp against torch's headers; returns a
    function (seed, stream, block) list -> list of 4-word tuples."""
    import torch.utils.cpp_extension as ce
    exe = os.path.join(str(outdir), "philox_torch_ref")
    inc = sum((["-I", p] for p in ce.include_paths()), [])
    subprocess.run(["g++", "-std=c++17", "-O1", *inc, "-o", exe,
                    os.path.join(HERE, "philox_torch_ref.cpp")], check=True)

    def run(triples):
        text = "".join(f"{s} {st} {b}\n" for s, st, b in triples)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [tuple(int(w) for w in line.split()) for line in out.splitlines()]
    return run


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    return build_torch_philox(tmp_path_factory.mktemp("philox"))


def test_philox_block_matches_torch_engine(olib, torch_philox):
    rnd = random.Random(1234)
    m64 = (1 << 64) - 1
    triples = [(0, 0, 0), (m64, m64, m64), (1, 0, 0), (0, 1, 0), (0, 0, 1)]
    triples += [(rnd.getrandbits(64), rnd.getrandbits(64), rnd.getrandbits(64)) for _ in range(300)]
    triples += [(0, off, blk) for off in (0, 1, 7) for blk in range(64)]
    want = torch_philox(triples)
    for (seed, stream, block), w in zip(triples, want):
        ctr = [block & 0xFFFFFFFF, block >> 32, stream & 0xFFFFFFFF, stream >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        got = tuple(int(v) for v in oracle.philox4x32_10(ctr, key, L=olib))
        assert got == w, (seed, stream, block)


def test_dropout_word_selects_word_e_mod_4_of_block_e_div_4(olib, torch_philox):
    rnd = random.Random(99)
    cases = [(rnd.getrandbits(64), rnd.randrange(4), rnd.getrandbits(40)) for _ in range(200)]
    want = torch_philox([(s, o, e // 4) for s, o, e in cases])
    for (s, o, e), w in zip(cases, want):
        assert oracle.dropout_word(s, o, e, L=olib) == w[e % 4]


def test_threshold_is_floor_p_times_2_pow_32_exactly(olib):
    for p in [0.0, 0.1, 0.5, 0.25, 1e-7, 0.9999999, 0.3, 0.05]:
        pf = np.float32(p)
        want = int(Fraction(float(pf)) * (1 << 32))          # floor of an exact rational
        assert oracle.dropout_threshold(float(pf), L=olib) == want
    assert oracle.dropout_threshold(0.1, L=olib) == 429496736


def test_scale_is_reciprocal_of_keep_probability(olib):
    for p in [0.0, 0.1, 0.5, 0.25, 0.3, 0.9]:
        pf = np.float32(p)
        exact = 1 / (1 - Fraction(float(pf)))
        got = oracle.dropout_scale(float(pf), L=olib)
        ulp = np.spacing(np.float32(got))
        assert abs(Fraction(got) - exact) <= Fraction(float(ulp)) / 2
    assert oracle.dropout_scale(0.0, L=olib) == 1.0


def _special_floats():
    vals = [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 3.3895313e38, 3.4028235e38,
            np.inf, -np.inf, 1e-40, -1e-40, 1.17549435e-38, 65504.0, 1.0 / 3]
    # exact ties: low 16 bits == 0x8000, kept lsb even and odd
    for hi in (0x3F80, 0x3F81, 0x4049, 0xC049, 0x0001, 0x7F7F):
        vals.append(np.array([(hi << 16) | 0x8000], np.uint32).view(np.float32)[0])
        vals.append(np.array([(hi << 16) | 0x7FFF], np.uint32).view(np.float32)[0])
        vals.append(np.array([(hi << 16) | 0x8001], np.uint32).view(np.float32)[0])
    return np.array(vals, np.float32)


def test_bf16_rounding_matches_torch(olib):
    import torch
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        _special_floats(),
        rng.standard_normal(20000, dtype=np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    vals = vals[~np.isnan(vals)]
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(vals, L=olib)
    assert np.array_equal(got, want)


def test_bf16_nan_stays_nan_and_widening_is_exact(olib):
    nan = np.array([0x7FC00001, 0xFF800001, 0x7F800001], np.uint32).view(np.float32)
    for v in nan:
        b = int(oracle.f32_to_bf16([v], L=olib)[0])
        assert (b & 0x7F80) == 0x7F80 and (b & 0x007F) != 0
    # every non-NaN pattern (a NaN would be quieted by the ctypes float return)
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits & 0x7F80) != 0x7F80) | ((bits & 0x007F) == 0)][::7]
    wide = np.array([olib.spo_bf16_to_f32(int(b)) for b in bits], np.float32)
    ref = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(wide.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------- mask statistics
def _mask(olib, rows, h, p, seed=0, offset=0, shard_index=0, t=1):
    d = oracle.Desc(s_local=rows, b=1, h=h, shard_index=shard_index, t=t, io=oracle.F32,
                    norm=oracle.LAYERNORM, p=p, eps=1e-5, seed=seed, offset=offset)
    z = np.zeros(rows * h, np.float32)
    out = oracle.fwd(d, z, None, z, np.ones(h, np.float32), np.zeros(h, np.float32), L=olib)
    return out["mask"].reshape(rows, h)


def test_mask_matches_library_words_and_global_index(olib, torch_philox):
    # Shard 1 of 2 of a [8, 1, 16] tensor: its element (r, c) is global
    # element (8 + r) * 16 + c of the full tensor.
    p = np.float32(0.3)
    m = _mask(olib, rows=8, h=16, p=float(p), seed=5, offset=3, shard_index=1, t=2)
    thr = int(Fraction(float(p)) * (1 << 32))
    es = [(8 + r) * 16 + c for r in range(8) for c in range(16)]
    words = torch_philox([(5, 3, e // 4) for e in es])
    want = np.array([w[e % 4] >= thr for e, w in zip(es, words)], np.uint8).reshape(8, 16)
    assert np.array_equal(m, want)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_kept_fraction_and_uniformity(olib, p):
    rows, h = 2048, 256
    m = _mask(olib, rows, h, p, seed=11, offset=0)
    n = m.size
    q = 1.0 - oracle.dropout_threshold(p, L=olib) / 2**32
    sigma = np.sqrt(n * q * (1 - q))
    assert abs(m.sum() - n * q) < 5 * sigma
    # per-column and per-row kept counts: chi-square against the binomial
    for counts, k in ((m.sum(axis=0), rows), (m.sum(axis=1), h)):
        var = k * q * (1 - q)
        chi2 = float(((counts - k * q) ** 2 / var).sum())
        dof = counts.size
        assert abs(chi2 - dof) < 5 * np.sqrt(2 * dof)


def test_different_offsets_and_seeds_give_independent_masks(olib):
    p, rows, h = 0.1, 1024, 256
    a = _mask(olib, rows, h, p, seed=3, offset=0)
    b = _mask(olib, rows, h, p, seed=3, offset=1)
    c = _mask(olib, rows, h, p, seed=4, offset=0)
    n = a.size
    q = 1.0 - oracle.dropout_threshold(p, L=olib) / 2**32
    expect = 2 * q * (1 - q)
    for other in (b, c):
        dis = float((a != other).mean())
        assert abs(dis - expect) < 5 * np.sqrt(expect * (1 - expect) / n)

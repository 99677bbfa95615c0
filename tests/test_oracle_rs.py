"""Pins of the oracle's reduce-scatter prologue (spo_reduce_parts):
x = round_io(parts[0] + parts[1] + ... in rank order, fp32 adds).

Each pin is fixed by arithmetic, not by re-typing the oracle: the identity
at one part, exact integer sums, a case whose fp32 result depends on the
order of the adds, and ties of the final bf16 rounding."""
import numpy as np
import pytest

import oracle

F32, BF16 = oracle.F32, oracle.BF16


def _desc(n_elems, io, h=4):
    assert n_elems % h == 0
    return oracle.Desc(s_local=n_elems // h, b=1, h=h, io=io)


def _to_io(values, io):
    v = np.asarray(values, np.float32)
    if io == F32:
        return v
    bits = v.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "test values must be exact in bf16"
    return (bits >> 16).astype(np.uint16)


def _from_io(x, io):
    return np.asarray(x, np.float32) if io == F32 else oracle.bf16_to_f32(x)


@pytest.mark.parametrize("io", [F32, BF16])
def test_one_part_is_the_identity(olib, io):
    rng = np.random.default_rng(3)
    v = rng.standard_normal(64).astype(np.float32)
    if io == BF16:
        v = oracle.bf16_to_f32(oracle.f32_to_bf16(v, L=olib))
    x = oracle.reduce_parts(_desc(64, io), _to_io(v, io), L=olib)
    assert np.array_equal(_from_io(x, io), v)


@pytest.mark.parametrize("io,nparts", [(F32, 2), (F32, 8), (BF16, 4), (BF16, 8)])
def test_integer_parts_sum_exactly(olib, io, nparts):
    # small integers: every partial sum is exact in fp32 and the total
    # (|sum| <= 8 * 15 = 120 < 256) is exact in bf16, so x is the integer sum
    rng = np.random.default_rng(nparts)
    ints = rng.integers(-15, 16, size=(nparts, 32))
    x = oracle.reduce_parts(_desc(32, io), _to_io(ints.astype(np.float32).ravel(), io), L=olib)
    assert np.array_equal(_from_io(x, io), ints.sum(axis=0).astype(np.float32))


@pytest.mark.parametrize("io", [F32, BF16])
def test_parts_are_added_in_rank_order(olib, io):
    # 1 + 2^-24 is a tie that rounds back to 1 (even), so in rank order the
    # three small parts vanish one by one: x = 1.  Added smallest first, they
    # would sum to 3 * 2^-24 and survive (1 + 2^-22 in fp32).
    tiny = 2.0 ** -24
    parts = np.array([[1.0, 0.0, 0.0, 1.0], [tiny, tiny, 1.0, tiny],
                      [tiny, tiny, tiny, tiny], [tiny, tiny, tiny, tiny]], np.float32)
    x = oracle.reduce_parts(_desc(4, io), _to_io(parts.ravel(), io), L=olib)
    got = _from_io(x, io)
    assert got[0] == 1.0 and got[3] == 1.0
    assert got[1] == np.float32(3 * tiny)                 # exact in fp32 and bf16
    assert got[2] == 1.0
    # the reversed order gives a different fp32 sum: the pin has teeth
    rev = np.float32(tiny) + np.float32(tiny) + np.float32(tiny) + np.float32(1.0)
    assert rev != np.float32(1.0)


def test_bf16_final_rounding_is_one_rne(olib):
    # fp32 sums that fall exactly between two bf16 values (ulp 2^-7 at 1):
    # 1 + 2^-8 -> 1 (even), (1 + 2^-7) + 2^-8 -> 1 + 2^-6 (even), and
    # 1 + 2^-8 + 2^-9 (above the tie) -> 1 + 2^-7.  Rounding after each add
    # (bf16 accumulation) would give 1 for the last case.
    a, b, c = 2.0 ** -7, 2.0 ** -8, 2.0 ** -9
    parts = np.array([[1.0, 1.0 + a, 1.0, 1.0], [b, b, b, 0.0], [0.0, 0.0, c, 0.0]], np.float32)
    x = oracle.reduce_parts(_desc(4, BF16), _to_io(parts.ravel(), BF16), L=olib)
    assert list(_from_io(x, BF16)) == [1.0, 1.0 + 2.0 ** -6, 1.0 + a, 1.0]


def test_rejects_bad_arguments(olib):
    d = _desc(8, F32)
    with pytest.raises(ValueError):
        oracle.reduce_parts(d, np.zeros(12, np.float32), L=olib)

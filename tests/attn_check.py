"""Comparison rule between the GPU ring-attention forward and the oracle's
ordinary attention ("Sequence parallel math", section "Context parallelism
and ring attention": after the t ring steps every query has attended every
key, so the result is attention over all of them).

The bounds follow from the kernel's arithmetic.  With w_j the oracle's
softmax weights of one query over every key j and v_j the values of one
output dimension:

* The probabilities p_j enter P V rounded to bf16 (8 significant bits: a
  relative error d_j with |d_j| <= 2^-8); the row sum l adds the unrounded
  fp32 p_j.  O = sum_j w_j (1 + d_j) v_j, so |dO| <= 2^-8 * A with
  A = sum_j w_j |v_j| -- the oracle's attention over |V| (exact: |v| of a
  bf16 value is a bf16 value).
* The scores are fp32 sums of d exact bf16 products: each is off by at most
  eta_j = scale * g_d * sum_i |q_i k_ji| (g_d = d u / (1 - d u), u = 2^-24),
  which moves the weights by a factor within exp(+-2 eta) and O by at most
  2 (e^(2 eta) - 1) A, eta the largest eta_j of the query.
* fp32 accumulation of P V and of l over at most 2^16 keys, the rescales
  and the merge: at most 2^-12 * A.
* O is rounded to bf16 once: ulp_bf16(O).
Per element:  |O_gpu - O| <= ulp_bf16(O) + (2^-8 + 2^-12 + 2 (e^(2 eta) - 1)) A.

Those are worst cases (every rounding aligned with sign(v_j)).  The errors
are in fact random, so a second check bounds the mean square error by its
expectation: E[d_j^2] <= 2^-16 / 3 for round-to-nearest to 8 bits, so per
element E[dO^2] <= 2^-16/3 * sum_j w_j^2 v_j^2 + ulp_bf16(O)^2 / 12, plus the
fp32 and score terms above taken as (2^-14 A)^2 and ((e^(2 eta) - 1) A)^2.
The mean of dO^2 over the checked elements must stay within 4 times the mean
of that bound.  A misplaced key in the V^T layout moves O by
(w_a - w_b)(v_b - v_a) per tile, which this second check sees even when the
weights are spread over thousands of keys.

lse (fp32): |lse_gpu - lse| <= 1e-4 + 1e-5 |lse|.
"""
import numpy as np

import oracle
from tests import parity as P

U = 2.0 ** -24


def _f(bits):
    return oracle.bf16_to_f32(bits).astype(np.float64)


def check_attention(name, od, q, k, v, got_o, got_lse, want_o, want_lse, rows=None):
    """od: the oracle's AttnDesc; q: the query tokens `rows` (default all) as
    bf16 bits; k, v: every block's keys and values as bf16 bits; got_*: the
    GPU's O (bf16 bits) and lse (fp32 or None); want_*: the oracle's."""
    r0, r1 = rows if rows is not None else (0, od.s_local)
    nq, bh, D = r1 - r0, od.b * od.heads, od.d
    T = od.t * od.s_local
    scale = float(np.float32(od.scale if od.scale > 0 else 1.0 / np.sqrt(od.d)))

    a_abs, _ = oracle.attention(od, q, k, np.asarray(v, np.uint16) & np.uint16(0x7FFF), rows=rows)
    Q = _f(q).reshape(nq, bh, D).transpose(1, 0, 2)          # [bh, nq, D]
    K = _f(k).reshape(T, bh, D).transpose(1, 2, 0)           # [bh, D, T]
    V = _f(v).reshape(T, bh, D).transpose(1, 0, 2)           # [bh, T, D]
    g_d = D * U / (1.0 - D * U)
    eta = scale * g_d * np.matmul(np.abs(Q), np.abs(K)).max(axis=2)      # [bh, nq]
    s = scale * np.matmul(Q, K)                                           # [bh, nq, T]
    w = np.exp(s - s.max(axis=2, keepdims=True))
    w /= w.sum(axis=2, keepdims=True)
    w2v2 = np.matmul(w * w, V * V)                                        # [bh, nq, D]
    to_flat = lambda a: a.transpose(1, 0, 2).reshape(-1)                  # -> [nq, bh, D]
    eta_e = to_flat(np.broadcast_to(eta[:, :, None], (bh, nq, D)))
    w2v2 = to_flat(w2v2)

    o = oracle.bf16_to_f32(got_o).astype(np.float64)
    err = np.abs(o - want_o)
    ulp = P.ulp_bf16(want_o)
    score = np.expm1(2.0 * eta_e)
    bound = ulp + (2.0 ** -8 + 2.0 ** -12 + 2.0 * score) * a_abs
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (f"{name}: {bad.size} of {err.size} outside the bound; first at "
                           f"{bad[0]}: {o[bad[0]]} vs {want_o[bad[0]]} (bound {bound[bad[0]]:.3g})")
    mse_bound = (2.0 ** -16 / 3.0 * w2v2 + ulp ** 2 / 12.0 + (2.0 ** -14 * a_abs) ** 2
                 + (score * a_abs) ** 2)
    mse = float(np.mean(err ** 2))
    assert mse <= 4.0 * float(np.mean(mse_bound)), (
        f"{name}: rms error {np.sqrt(mse):.3g} above twice its expected "
        f"{np.sqrt(np.mean(mse_bound)):.3g}")
    if got_lse is not None:
        lerr = np.abs(np.asarray(got_lse, np.float64) - want_lse)
        assert np.all(lerr <= 1e-4 + 1e-5 * np.abs(want_lse)), f"{name}: lse off by {lerr.max()}"

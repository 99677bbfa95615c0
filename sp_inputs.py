"""Seeded synthetic inputs for the sequence-parallel region, and the workloads.

This module only draws numbers; it holds none of the region's arithmetic.
It is shared by the oracle-side and the GPU-side checks so that both read
identical bits.

Recipe (the pages measure on no dataset; activations are synthetic by nature):
  numpy.random.default_rng(seed) (PCG64), standard_normal in float32, drawn
  in this fixed order over the FULL [s, b, h] tensor (rows = s*b, row-major):
    x (the reduced row-parallel output), residual, dy (gradient of y),
    [dh_out], bias * 0.02, beta * 0.02, gamma = 1 + 0.02 * noise.
  "N(0, 0.02)" is read as standard deviation 0.02.  bf16 tensors are the
  round-to-nearest-even bfloat16 of those float32 draws, made by torch's
  float32 -> bfloat16 conversion, and travel as raw uint16 bit patterns.
  Shard i of t is rows [i*s/t*b, (i+1)*s/t*b) of the full tensor (the
  sequence-major layout makes a shard one contiguous slab).
  The partial slabs of the reduce-scatter prologue (make_parts): a second
  generator, default_rng(seed + 1), draws nparts slabs of standard normals
  in rank order, each scaled by 1/sqrt(nparts) so that their sum has the
  unit variance of x.
  Ring attention (make_attn_inputs): default_rng(seed + 2) draws q, then k
  and v of all t blocks, standard normals rounded to bf16.
  The matched-key attention inputs (make_attn_inputs_matched) come from
  default_rng(seed + 4); see that function.
"""
from dataclasses import dataclass, field

import numpy as np

F32, BF16 = 0, 1
LAYERNORM, RMSNORM = 0, 1


def to_bf16_bits(a32):
    """float32 array -> raw bfloat16 patterns (uint16), RNE, via torch."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make_inputs(rows, h, io, seed=0, dh_out=False):
    """Draws every input of one region call over `rows` token rows of width h.

    Returns a dict of numpy arrays: x, residual, dy, dh_out (or None) in the
    I/O type (float32 or uint16 bf16 bits), and bias, beta, gamma in float32.
    """
    rng = np.random.default_rng(seed)
    n = rows * h
    std = lambda k: rng.standard_normal(k, dtype=np.float32)
    x, residual, dy = std(n), std(n), std(n)
    dho = std(n) if dh_out else None
    bias = std(h) * np.float32(0.02)
    beta = std(h) * np.float32(0.02)
    gamma = np.float32(1.0) + std(h) * np.float32(0.02)
    cast = to_bf16_bits if io == BF16 else (lambda a: a)
    return {"x": cast(x), "residual": cast(residual), "dy": cast(dy),
            "dh_out": None if dho is None else cast(dho),
            "bias": bias, "beta": beta, "gamma": gamma}


def make_parts(rows, h, io, nparts, seed=0):
    """nparts partial slabs [nparts, rows*h] of the row-parallel output, in
    the I/O type (see the module recipe)."""
    rng = np.random.default_rng(seed + 1)
    scale = np.float32(1.0 / np.sqrt(nparts))
    parts = rng.standard_normal((nparts, rows * h), dtype=np.float32) * scale
    return to_bf16_bits(parts) if io == BF16 else parts


def make_attn_inputs(s_local, b, heads, d, t, seed=0):
    """Ring attention: this rank's queries q [s_local*b*heads*d] and the
    keys/values of all t blocks k, v [t*s_local*b*heads*d], standard normals
    from default_rng(seed + 2) drawn in the order q, k, v, as bf16 bits."""
    rng = np.random.default_rng(seed + 2)
    n = s_local * b * heads * d
    q = rng.standard_normal(n, dtype=np.float32)
    k = rng.standard_normal(t * n, dtype=np.float32)
    v = rng.standard_normal(t * n, dtype=np.float32)
    return {"q": to_bf16_bits(q), "k": to_bf16_bits(k), "v": to_bf16_bits(v)}


def make_attn_inputs_ramp(s_local, b, heads, d, t, seed=0, span=200.0, rising=True):
    """Ring attention whose scores climb (rising) or fall steadily along the
    global key index j of the S = t * s_local key tokens: every element of q
    is 1 + 0.05 N(0,1); key j is g_j (1 + 0.05 N(0,1)) per element with
    g_j = c j / (S - 1) (rising) or c (S - 1 - j) / (S - 1), c chosen so that
    the scaled scores q.k / sqrt(d) span about `span` in base-2 units; v is
    standard normal.  Drawn from default_rng(seed + 3) in the order q, k, v,
    as bf16 bits.  A streaming softmax must move its reference many times on
    such keys (or, falling, almost never)."""
    rng = np.random.default_rng(seed + 3)
    S = t * s_local
    n = s_local * b * heads * d
    c = span / (np.sqrt(d) * np.log2(np.e))
    q = 1.0 + 0.05 * rng.standard_normal(n)
    j = np.arange(S, dtype=np.float64)
    g = c * (j if rising else (S - 1 - j)) / max(S - 1, 1)
    k = (1.0 + 0.05 * rng.standard_normal((S, b * heads * d))) * g[:, None]
    v = rng.standard_normal(t * n)
    f = lambda a: to_bf16_bits(np.asarray(a, dtype=np.float32).reshape(-1))
    return {"q": f(q), "k": f(k), "v": f(v)}


def make_attn_inputs_matched(s_local, b, heads, d, t, seed=0, gain=4.0):
    """Ring attention in which every query has one key of its own that
    dominates its softmax: q is standard normal (rounded to bf16), every key
    starts as 0.5 N(0,1) and value as N(0,1); then, per (batch, head), query i
    is matched to key perm[i] (a random injection of the s_local queries into
    the t * s_local keys) and that key is set to gain * q_i (gain a power of
    two, so exact in bf16).  The matched score, gain |q_i|^2 / sqrt(d) ~
    gain sqrt(d), exceeds every other by ~20 or more, so the output is the
    matched key's value to within ~1e-6: a value read from the wrong key
    position moves it by O(1).  Drawn from default_rng(seed + 4) in the order
    q, k, v, perm, as bf16 bits."""
    rng = np.random.default_rng(seed + 4)
    S, T = s_local, t * s_local
    q = to_bf16_bits(rng.standard_normal((S, b, heads, d), dtype=np.float32))
    k = rng.standard_normal((T, b, heads, d), dtype=np.float32) * np.float32(0.5)
    v = rng.standard_normal(T * b * heads * d, dtype=np.float32)
    perm = rng.permutation(T)[:S]
    qf = (q.astype(np.uint32) << 16).view(np.float32)
    k[perm] = np.float32(gain) * qf
    return {"q": q.reshape(-1), "k": to_bf16_bits(k.reshape(-1)), "v": to_bf16_bits(v),
            "perm": perm}


@dataclass
class Workload:
    """One shard shape and region setting (sizes as the pages' layers)."""
    name: str
    s: int                 # full sequence length
    b: int                 # batch
    h: int                 # hidden size
    t: int                 # sequence/tensor-parallel degree
    io: int                # F32 or BF16
    norm: int              # LAYERNORM or RMSNORM
    p: float               # dropout probability
    eps: float
    a: int = 0             # attention heads (accounting only)
    seed: int = 0
    calls_per_layer: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def s_local(self):
        return self.s // self.t

    @property
    def rows(self):        # N = s/t * b token rows in one shard
        return self.s_local * self.b

    @property
    def elems(self):
        return self.rows * self.h


WORKLOADS = {
    # A tiny fp32 shard for exhaustive checks: [64, 2, 256] of [128, 2, 256].
    "tiny_fp32_t2": Workload("tiny_fp32_t2", s=128, b=2, h=256, t=2, io=F32,
                             norm=LAYERNORM, p=0.1, eps=1e-5),
    # 22B-class layer boundary (one layer of a 22B model): shard [256, 4, 6144].
    "22b_h6144_t8": Workload("22b_h6144_t8", s=2048, b=4, h=6144, t=8, io=BF16,
                             norm=LAYERNORM, p=0.1, eps=1e-5, a=64),
    # 175B-class (GPT-3-scale) layer boundary: shard [256, 8, 12288], two
    # region calls per layer (pre-attention and pre-MLP).
    "175b_h12288_t8": Workload("175b_h12288_t8", s=2048, b=8, h=12288, t=8, io=BF16,
                               norm=LAYERNORM, p=0.1, eps=1e-5, a=96, calls_per_layer=2),
    # Long-sequence RMSNorm variant: shard [4096, 1, 8192].
    "longseq_rms_h8192_t8_p0.1": Workload("longseq_rms_h8192_t8_p0.1", s=32768, b=1, h=8192,
                                          t=8, io=BF16, norm=RMSNORM, p=0.1, eps=1e-6),
    "longseq_rms_h8192_t8_p0": Workload("longseq_rms_h8192_t8_p0", s=32768, b=1, h=8192,
                                        t=8, io=BF16, norm=RMSNORM, p=0.0, eps=1e-6),
    # 1T-class wide rows, shard-size sweep t in {1, 2, 4, 8}: [2048/t, 4, 25600].
    **{f"1t_h25600_t{t}": Workload(f"1t_h25600_t{t}", s=2048, b=4, h=25600, t=t, io=BF16,
                                   norm=LAYERNORM, p=0.1, eps=1e-5, a=160, calls_per_layer=2)
       for t in (1, 2, 4, 8)},
}

HEADLINE = "22b_h6144_t8"


@dataclass
class AttnWorkload:
    """One rank of a ring-attention forward: s tokens split over t ranks,
    `heads` heads of width d on this GPU (the model's heads divided by the
    tensor-parallel degree)."""
    name: str
    s: int
    t: int
    b: int
    heads: int
    d: int
    seed: int = 0

    @property
    def s_local(self):
        return self.s // self.t

    @property
    def flops(self):
        """Multiply-adds x 2 of Q K^T and P V over all keys."""
        return 4 * self.s_local * self.s * self.b * self.heads * self.d


ATTN_WORKLOADS = {
    # The long-sequence configuration's attention core under context
    # parallelism: s = 32768 over t = 8 ranks, h = 8192 = 64 heads of 128,
    # 8 of them per GPU (tensor-parallel degree 8).
    "ring_attn_s32k_t8_h8192": AttnWorkload("ring_attn_s32k_t8_h8192", s=32768, t=8, b=1,
                                            heads=8, d=128),
    # The same heads at the 22B layer's length: s = 2048 over t = 8.
    "ring_attn_s2k_t8_d128": AttnWorkload("ring_attn_s2k_t8_d128", s=2048, t=8, b=4, heads=8,
                                          d=128),
}

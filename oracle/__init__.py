"""numpy front end of the CPU oracle (oracle/libsp_oracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and
the CPU-baseline leg of bench.py, never by the product package.  It does
argument marshalling only; every step of the computation is in sp_oracle.c.

Arrays: fp32 I/O tensors are numpy float32, bf16 I/O tensors are numpy
uint16 holding the raw bfloat16 bit patterns; parameters and statistics are
float32; masks are uint8 (1 = keep).
"""
import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsp_oracle.so")

F32, BF16 = 0, 1
LAYERNORM, RMSNORM = 0, 1


class _Desc(ctypes.Structure):
    _fields_ = [("s_local", ctypes.c_int64), ("b", ctypes.c_int64), ("h", ctypes.c_int64),
                ("shard_index", ctypes.c_int32), ("t", ctypes.c_int32),
                ("io", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("p", ctypes.c_float), ("eps", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


@dataclass
class Desc:
    """One rank's shard [s_local, b, h] and the region's settings."""
    s_local: int
    b: int
    h: int
    shard_index: int = 0
    t: int = 1
    io: int = F32
    norm: int = LAYERNORM
    p: float = 0.0
    eps: float = 1e-5
    seed: int = 0
    offset: int = 0

    @property
    def rows(self):
        return self.s_local * self.b

    def c(self):
        return _Desc(self.s_local, self.b, self.h, self.shard_index, self.t, self.io,
                     self.norm, self.p, self.eps, self.seed, self.offset)


_lib = None


def lib():
    """Loads the oracle library (build it with oracle/build.py first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"oracle library missing: {LIB_PATH}; run oracle/build.py")
        _lib = load(LIB_PATH)
    return _lib


def load(path):
    """Loads an oracle build at `path` and declares its signatures."""
    L = ctypes.CDLL(path)
    P, I64, U64, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32
    D = ctypes.POINTER(_Desc)
    L.spo_philox4x32_10.argtypes = [P, P, P]
    L.spo_philox4x32_10.restype = None
    L.spo_dropout_word.argtypes = [U64, U64, U64]
    L.spo_dropout_word.restype = U32
    L.spo_dropout_threshold.argtypes = [ctypes.c_float]
    L.spo_dropout_threshold.restype = U32
    L.spo_dropout_scale.argtypes = [ctypes.c_float]
    L.spo_dropout_scale.restype = ctypes.c_float
    L.spo_f32_to_bf16.argtypes = [ctypes.c_float]
    L.spo_f32_to_bf16.restype = ctypes.c_uint16
    L.spo_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.spo_bf16_to_f32.restype = ctypes.c_float
    L.spo_attention.argtypes = [ctypes.POINTER(spo_attn_desc), I64, I64, P, P, P, P, P]
    L.spo_attention.restype = ctypes.c_int
    L.spo_reduce_parts.argtypes = [D, ctypes.c_int, P, P]
    L.spo_reduce_parts.restype = ctypes.c_int
    L.spo_fwd.argtypes = [D, I64, I64] + [P] * 10
    L.spo_fwd.restype = ctypes.c_int
    L.spo_bwd.argtypes = [D, I64, I64] + [P] * 12
    L.spo_bwd.restype = ctypes.c_int
    L.spo_fwd_exact.argtypes = [D] + [P] * 10
    L.spo_fwd_exact.restype = ctypes.c_int
    L.spo_bwd_exact.argtypes = [D] + [P] * 12
    L.spo_bwd_exact.restype = ctypes.c_int
    L.spo_activation_bytes.argtypes = [D, P, P]
    L.spo_activation_bytes.restype = ctypes.c_int
    L.spo_layer_activation_elems.argtypes = [ctypes.c_double] * 5 + [P, P, P]
    L.spo_layer_activation_elems.restype = None
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _io_dtype(d):
    return np.uint16 if d.io == BF16 else np.float32


def _check(a, dtype, n, name):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype or a.size != n:
        raise ValueError(f"{name}: want {n} x {np.dtype(dtype).name}, got {a.size} x {a.dtype}")
    return a


# ---------------------------------------------------------------- generator
def philox4x32_10(ctr, key, L=None):
    L = L or lib()
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    L.spo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def dropout_word(seed, offset, e, L=None):
    return int((L or lib()).spo_dropout_word(seed, offset, e))


def dropout_threshold(p, L=None):
    return int((L or lib()).spo_dropout_threshold(p))


def dropout_scale(p, L=None):
    return float((L or lib()).spo_dropout_scale(p))


def f32_to_bf16(values, L=None):
    L = L or lib()
    v = np.asarray(values, dtype=np.float32).ravel()
    return np.array([L.spo_f32_to_bf16(float(f)) for f in v], dtype=np.uint16)


def bf16_to_f32(bits):
    """Exact widening of raw bf16 patterns (a shift; no rounding involved)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- ring attention
class spo_attn_desc(ctypes.Structure):
    _fields_ = [("s_local", ctypes.c_int64), ("b", ctypes.c_int64), ("heads", ctypes.c_int32),
                ("d", ctypes.c_int32), ("t", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("scale", ctypes.c_float)]


@dataclass
class AttnDesc:
    """One rank of a ring of t: s_local query tokens, K/V blocks of s_local
    tokens each; [tokens, b, heads, d] layouts."""
    s_local: int
    b: int
    heads: int
    d: int
    t: int = 1
    rank: int = 0
    scale: float = 0.0          # 0: 1/sqrt(d)

    def c(self):
        sc = self.scale if self.scale > 0 else 1.0 / np.sqrt(self.d)
        return spo_attn_desc(self.s_local, self.b, self.heads, self.d, self.t, self.rank, sc)


def attention(d, q, k, v, rows=None, L=None):
    """Ordinary attention of the rank's queries over the keys of all t
    blocks, float64.  q: the query tokens [r0, r1) (default: all s_local)
    as bf16 bits; k, v: all t blocks.  Returns (o float64, lse float64) for
    those queries."""
    L = L or lib()
    r0, r1 = rows if rows is not None else (0, d.s_local)
    tok = d.b * d.heads * d.d
    q = _check(q, np.uint16, (r1 - r0) * tok, "q")
    k = _check(k, np.uint16, d.t * d.s_local * tok, "k")
    v = _check(v, np.uint16, d.t * d.s_local * tok, "v")
    o = np.empty((r1 - r0) * tok, np.float64)
    lse = np.empty((r1 - r0) * d.b * d.heads, np.float64)
    if L.spo_attention(ctypes.byref(d.c()), r0, r1, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                       _ptr(lse)) != 0:
        raise ValueError("spo_attention rejected its arguments")
    return o, lse


# ---------------------------------------------------------------- region
def reduce_parts(d, parts, L=None):
    """x = round_io(parts[0] + parts[1] + ... in that order, fp32 adds).
    parts: array of nparts * N * h I/O elements ([nparts][N][h])."""
    L = L or lib()
    io = _io_dtype(d)
    n = d.rows * d.h
    parts = np.ascontiguousarray(parts, dtype=io).ravel()
    if parts.size % n != 0 or parts.size == 0:
        raise ValueError("parts must hold nparts * N * h elements")
    x = np.empty(n, io)
    if L.spo_reduce_parts(ctypes.byref(d.c()), parts.size // n, _ptr(parts), _ptr(x)) != 0:
        raise ValueError("spo_reduce_parts rejected its arguments")
    return x


def fwd(d, x, bias, residual, gamma, beta, rows=None, L=None, write_h=True):
    """Forward over rows [r0, r1) (default: the whole shard).  x and residual
    hold exactly those rows.  Returns dict h, y, mask, mean, rstd.
    x = None: the norm-only entry (h is the residual; write_h=False leaves
    h unwritten, returned as None); gamma = None: the norm-free exit (h and
    mask only)."""
    L = L or lib()
    r0, r1 = rows if rows is not None else (0, d.rows)
    n, H, io = r1 - r0, d.h, _io_dtype(d)
    x = _check(x, io, n * H, "x")
    residual = _check(residual, io, n * H, "residual")
    bias = _check(bias, np.float32, H, "bias")
    gamma = _check(gamma, np.float32, H, "gamma")
    beta = _check(beta, np.float32, H, "beta")
    norm = gamma is not None
    out = {"h": np.empty(n * H, io) if (x is not None or write_h) else None,
           "y": np.empty(n * H, io) if norm else None,
           "mask": np.empty(n * H, np.uint8) if d.p > 0 and x is not None else None,
           "mean": np.empty(n, np.float32) if norm and d.norm == LAYERNORM else None,
           "rstd": np.empty(n, np.float32) if norm else None}
    rc = L.spo_fwd(ctypes.byref(d.c()), r0, r1, _ptr(x), _ptr(bias), _ptr(residual),
                   _ptr(gamma), _ptr(beta), _ptr(out["h"]), _ptr(out["y"]),
                   _ptr(out["mask"]), _ptr(out["mean"]), _ptr(out["rstd"]))
    if rc != 0:
        raise ValueError("spo_fwd rejected its arguments")
    return out


def bwd(d, dy, dh_out, h, mask, mean, rstd, gamma, want_dbias=True, rows=None, L=None,
        want_dx=True, want_dres=True):
    """Backward over rows [r0, r1).  Returns dict dx, dres, dgamma, dbeta,
    dbias (parameter gradients are partial sums over those rows).
    dy = None: the norm-free exit (dh = dh_out; no dgamma/dbeta)."""
    L = L or lib()
    r0, r1 = rows if rows is not None else (0, d.rows)
    n, H, io = r1 - r0, d.h, _io_dtype(d)
    dy = _check(dy, io, n * H, "dy")
    dh_out = _check(dh_out, io, n * H, "dh_out")
    h = _check(h, io, n * H, "h")
    mask = _check(mask, np.uint8, n * H, "mask")
    mean = _check(mean, np.float32, n, "mean")
    rstd = _check(rstd, np.float32, n, "rstd")
    gamma = _check(gamma, np.float32, H, "gamma")
    norm = dy is not None
    out = {"dx": np.empty(n * H, io) if want_dx else None,
           "dres": np.empty(n * H, io) if want_dres else None,
           "dgamma": np.empty(H, np.float32) if norm else None,
           "dbeta": np.empty(H, np.float32) if norm and d.norm == LAYERNORM else None,
           "dbias": np.empty(H, np.float32) if want_dbias else None}
    rc = L.spo_bwd(ctypes.byref(d.c()), r0, r1, _ptr(dy), _ptr(dh_out), _ptr(h), _ptr(mask),
                   _ptr(mean), _ptr(rstd), _ptr(gamma), _ptr(out["dx"]), _ptr(out["dres"]),
                   _ptr(out["dgamma"]), _ptr(out["dbeta"]), _ptr(out["dbias"]))
    if rc != 0:
        raise ValueError("spo_bwd rejected its arguments")
    return out


def fwd_exact(d, x, bias, residual, gamma, beta, L=None):
    """All-float64 forward of the whole shard (no I/O rounding)."""
    L = L or lib()
    N, H = d.rows, d.h
    f8 = lambda a, n: _check(None if a is None else np.asarray(a, np.float64), np.float64, n, "arg")
    x, residual = f8(x, N * H), f8(residual, N * H)
    bias, gamma, beta = f8(bias, H), f8(gamma, H), f8(beta, H)
    out = {"h": np.empty(N * H), "y": np.empty(N * H),
           "mask": np.empty(N * H, np.uint8) if d.p > 0 else None,
           "mean": np.empty(N) if d.norm == LAYERNORM else None, "rstd": np.empty(N)}
    rc = L.spo_fwd_exact(ctypes.byref(d.c()), _ptr(x), _ptr(bias), _ptr(residual), _ptr(gamma),
                         _ptr(beta), _ptr(out["h"]), _ptr(out["y"]), _ptr(out["mask"]),
                         _ptr(out["mean"]), _ptr(out["rstd"]))
    if rc != 0:
        raise ValueError("spo_fwd_exact rejected its arguments")
    return out


def bwd_exact(d, dy, dh_out, h, mask, mean, rstd, gamma, L=None):
    """All-float64 backward of the whole shard."""
    L = L or lib()
    N, H = d.rows, d.h
    f8 = lambda a, n: _check(None if a is None else np.asarray(a, np.float64), np.float64, n, "arg")
    dy, dh_out, h = f8(dy, N * H), f8(dh_out, N * H), f8(h, N * H)
    mean, rstd, gamma = f8(mean, N), f8(rstd, N), f8(gamma, H)
    mask = _check(mask, np.uint8, N * H, "mask")
    out = {"dx": np.empty(N * H), "dres": np.empty(N * H), "dgamma": np.empty(H),
           "dbeta": np.empty(H) if d.norm == LAYERNORM else None, "dbias": np.empty(H)}
    rc = L.spo_bwd_exact(ctypes.byref(d.c()), _ptr(dy), _ptr(dh_out), _ptr(h), _ptr(mask),
                         _ptr(mean), _ptr(rstd), _ptr(gamma), _ptr(out["dx"]), _ptr(out["dres"]),
                         _ptr(out["dgamma"]), _ptr(out["dbeta"]), _ptr(out["dbias"]))
    if rc != 0:
        raise ValueError("spo_bwd_exact rejected its arguments")
    return out


# ---------------------------------------------------------------- accounting
def activation_bytes(d, L=None):
    L = L or lib()
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    if L.spo_activation_bytes(ctypes.byref(d.c()), ctypes.byref(a), ctypes.byref(b)) != 0:
        raise ValueError("spo_activation_bytes rejected its arguments")
    return a.value, b.value


def layer_activation_elems(s, b, h, a, t, L=None):
    L = L or lib()
    out = [ctypes.c_double() for _ in range(3)]
    L.spo_layer_activation_elems(s, b, h, a, t, *[ctypes.byref(o) for o in out])
    return tuple(o.value for o in out)

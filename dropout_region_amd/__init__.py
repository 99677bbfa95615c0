"""Python binding of libsp_region.so (include/sp_region.h).

Argument marshalling only: every step of the region runs in the library's
HIP kernels.  The functions carry the C names and take torch tensors (or
None) for the pointer arguments; torch provides device memory and the
current HIP stream.  There is no fallback: if the library is not built,
every call raises.
"""
import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsp_region.so")

SPR_OK, SPR_ERR_INVALID_ARG, SPR_ERR_UNSUPPORTED, SPR_ERR_WORKSPACE, SPR_ERR_HIP = range(5)
SPR_F32, SPR_BF16 = 0, 1
SPR_LAYERNORM, SPR_RMSNORM = 0, 1
SPR_FWD_AUTO, SPR_FWD_ROWS, SPR_FWD_STREAM = 0, 1, 2
SPR_BWD_AUTO, SPR_BWD_FUSED, SPR_BWD_SPLIT = 0, 1, 2


class SprError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {sp_region_status_string(status)} (status {status})")


class spr_desc(ctypes.Structure):
    _fields_ = [("s_local", ctypes.c_int64), ("b", ctypes.c_int64), ("h", ctypes.c_int64),
                ("shard_index", ctypes.c_int32), ("t", ctypes.c_int32),
                ("io", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("p", ctypes.c_float), ("eps", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64),
                ("fwd_kernel", ctypes.c_int32), ("bwd_path", ctypes.c_int32),
                ("bwd_tile_rows", ctypes.c_int32), ("reserved", ctypes.c_int32)]


@dataclass
class Desc:
    """Shard [s_local, b, h] of rank shard_index of t, region settings, and
    the launch choices (0: the library's own)."""
    s_local: int
    b: int
    h: int
    shard_index: int = 0
    t: int = 1
    io: int = SPR_BF16
    norm: int = SPR_LAYERNORM
    p: float = 0.0
    eps: float = 1e-5
    seed: int = 0
    offset: int = 0
    fwd_kernel: int = SPR_FWD_AUTO
    bwd_path: int = SPR_BWD_AUTO
    bwd_tile_rows: int = 0

    @property
    def rows(self):
        return self.s_local * self.b

    def c(self):
        return spr_desc(self.s_local, self.b, self.h, self.shard_index, self.t, self.io,
                        self.norm, self.p, self.eps, self.seed, self.offset, self.fwd_kernel,
                        self.bwd_path, self.bwd_tile_rows, 0)


class spr_attn_desc(ctypes.Structure):
    _fields_ = [("s_local", ctypes.c_int64), ("b", ctypes.c_int64), ("heads", ctypes.c_int32),
                ("d", ctypes.c_int32), ("t", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("scale", ctypes.c_float), ("steps_per_wg", ctypes.c_int32)]


@dataclass
class AttnDesc:
    """Ring attention on rank `rank` of t (include/sp_ring_attn.h)."""
    s_local: int
    b: int
    heads: int
    d: int
    t: int = 1
    rank: int = 0
    scale: float = 0.0
    steps_per_wg: int = 0       # launch choice: 0 = the library's own, else a divisor of t

    @property
    def rows(self):
        return self.s_local * self.b * self.heads

    def c(self):
        return spr_attn_desc(self.s_local, self.b, self.heads, self.d, self.t, self.rank,
                             self.scale, self.steps_per_wg)


_lib = None


def lib():
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build() or dropout_region_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P, D = ctypes.c_void_p, ctypes.POINTER(spr_desc)
        L.sp_region_fwd.argtypes = [D] + [P] * 10 + [P]
        L.sp_region_fwd.restype = ctypes.c_int
        L.sp_region_fwd_rs.argtypes = [D, P, ctypes.c_int32] + [P] * 9 + [P]
        L.sp_region_fwd_rs.restype = ctypes.c_int
        L.sp_region_bwd.argtypes = [D] + [P] * 12 + [P, ctypes.c_size_t, P]
        L.sp_region_bwd.restype = ctypes.c_int
        L.sp_region_bwd_noalloc.argtypes = [D] + [P] * 12 + [P]
        L.sp_region_bwd_noalloc.restype = ctypes.c_int
        L.sp_region_bwd_exit.argtypes = [D, P, P, P, P, P, ctypes.c_size_t, P]
        L.sp_region_bwd_exit.restype = ctypes.c_int
        L.sp_region_bwd_num_launches.argtypes = [D]
        L.sp_region_bwd_num_launches.restype = ctypes.c_int
        L.sp_region_bwd_launch.argtypes = [D, ctypes.c_int] + [P] * 12 + [P, ctypes.c_size_t, P]
        L.sp_region_bwd_launch.restype = ctypes.c_int
        L.sp_region_bwd_workspace_bytes.argtypes = [D]
        L.sp_region_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.sp_region_activation_bytes.argtypes = [D, P, P]
        L.sp_region_activation_bytes.restype = ctypes.c_int
        A = ctypes.POINTER(spr_attn_desc)
        L.sp_ring_attn_workspace_bytes.argtypes = [A]
        L.sp_ring_attn_workspace_bytes.restype = ctypes.c_size_t
        L.sp_ring_attn_fwd.argtypes = [A, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sp_ring_attn_fwd.restype = ctypes.c_int
        L.sp_ring_attn_step.argtypes = [A, ctypes.c_int32, P, P, P, P, ctypes.c_size_t, P]
        L.sp_ring_attn_step.restype = ctypes.c_int
        L.sp_ring_attn_merge.argtypes = [A, P, P, P, ctypes.c_size_t, P]
        L.sp_ring_attn_merge.restype = ctypes.c_int
        L.sp_ring_attn_fwd_num_launches.argtypes = [A]
        L.sp_ring_attn_fwd_num_launches.restype = ctypes.c_int
        L.sp_ring_attn_fwd_launch.argtypes = [A, ctypes.c_int, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sp_ring_attn_fwd_launch.restype = ctypes.c_int
        L.sp_region_status_string.argtypes = [ctypes.c_int]
        L.sp_region_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


# ------------------------------------------------------------ marshalling
def _io_dtype(d):
    import torch
    return torch.bfloat16 if d.io == SPR_BF16 else torch.float32


def _dev(t):
    """Device index of tensor t (-1 on the host), or None for no tensor."""
    return None if t is None else t.get_device()


def _arg(t, name, numel, dtype, device, optional=False):
    """Device pointer (an int for ctypes) of tensor t after checking what the
    C side cannot: device (an index, as _dev gives), dtype, contiguity and
    size.  Each check is one call into torch: this runs for every tensor of
    every call."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    g = t.get_device()
    if g < 0 or (device is not None and g != device):
        raise ValueError(f"{name} must be on GPU {device}")
    if t.dtype is not dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, want {dtype}")
    if not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name}: want a contiguous tensor of {numel} elements")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------ entry points
def sp_region_status_string(status):
    return lib().sp_region_status_string(int(status)).decode()


def sp_region_activation_bytes(d):
    """(saved_for_bwd, retained_output) bytes of one forward call."""
    a, b = ctypes.c_uint64(), ctypes.c_uint64()
    st = lib().sp_region_activation_bytes(ctypes.byref(d.c()), ctypes.byref(a), ctypes.byref(b))
    if st != SPR_OK:
        raise SprError("sp_region_activation_bytes", st)
    return a.value, b.value


def sp_region_bwd_workspace_bytes(d):
    return int(lib().sp_region_bwd_workspace_bytes(ctypes.byref(d.c())))


def sp_region_fwd(d, x, bias, residual, gamma, beta, h_out, y_out, mask_out, mean_out,
                  rstd_out, stream=None):
    import torch
    L = lib()
    N, H, io = d.rows, d.h, _io_dtype(d)
    dev = _dev(residual)
    f32, u8 = torch.float32, torch.uint8
    args = [_arg(x, "x", N * H, io, dev, True), _arg(bias, "bias", H, f32, dev, True),
            _arg(residual, "residual", N * H, io, dev), _arg(gamma, "gamma", H, f32, dev, True),
            _arg(beta, "beta", H, f32, dev, True), _arg(h_out, "h_out", N * H, io, dev, True),
            _arg(y_out, "y_out", N * H, io, dev, True),
            _arg(mask_out, "mask_out", N * H, u8, dev, True),
            _arg(mean_out, "mean_out", N, f32, dev, True),
            _arg(rstd_out, "rstd_out", N, f32, dev, True)]
    st = L.sp_region_fwd(ctypes.byref(d.c()), *args, _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_region_fwd", st)


def sp_region_fwd_rs(d, x_parts, nparts, bias, residual, gamma, beta, h_out, y_out, mask_out,
                     mean_out, rstd_out, stream=None):
    """sp_region_fwd with x = the sum of nparts partial slabs x_parts
    ([nparts, N, h], contiguous), added in the kernel's prologue."""
    import torch
    L = lib()
    N, H, io, dev = d.rows, d.h, _io_dtype(d), _dev(x_parts)
    f32, u8 = torch.float32, torch.uint8
    args = [_arg(x_parts, "x_parts", int(nparts) * N * H, io, dev), ctypes.c_int32(int(nparts)),
            _arg(bias, "bias", H, f32, dev, True),
            _arg(residual, "residual", N * H, io, dev), _arg(gamma, "gamma", H, f32, dev),
            _arg(beta, "beta", H, f32, dev, True), _arg(h_out, "h_out", N * H, io, dev),
            _arg(y_out, "y_out", N * H, io, dev), _arg(mask_out, "mask_out", N * H, u8, dev, True),
            _arg(mean_out, "mean_out", N, f32, dev, True), _arg(rstd_out, "rstd_out", N, f32, dev)]
    st = L.sp_region_fwd_rs(ctypes.byref(d.c()), *args, _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_region_fwd_rs", st)


def _bwd_args(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out, dgamma_out,
              dbeta_out, dbias_out, workspace):
    import torch
    N, H, io, dev = d.rows, d.h, _io_dtype(d), _dev(dy)
    f32, u8 = torch.float32, torch.uint8
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    return [_arg(dy, "dy", N * H, io, dev), _arg(dh_out, "dh_out", N * H, io, dev, True),
            _arg(h, "h", N * H, io, dev), _arg(mask, "mask", N * H, u8, dev, True),
            _arg(mean, "mean", N, f32, dev, True), _arg(rstd, "rstd", N, f32, dev),
            _arg(gamma, "gamma", H, f32, dev), _arg(dx_out, "dx_out", N * H, io, dev, True),
            _arg(dres_out, "dres_out", N * H, io, dev),
            _arg(dgamma_out, "dgamma_out", H, f32, dev),
            _arg(dbeta_out, "dbeta_out", H, f32, dev, True),
            _arg(dbias_out, "dbias_out", H, f32, dev, True),
            ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(ws_bytes)]


def sp_region_bwd(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out, dgamma_out,
                  dbeta_out, dbias_out, workspace, stream=None):
    args = _bwd_args(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out, dgamma_out,
                     dbeta_out, dbias_out, workspace)
    st = lib().sp_region_bwd(ctypes.byref(d.c()), *args, _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_region_bwd", st)


def sp_region_bwd_noalloc(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out,
                          dgamma_out, dbeta_out, dbias_out, stream=None):
    """sp_region_bwd with the library's own fixed scratch instead of a
    workspace (for callers that cannot allocate)."""
    import torch
    N, H, io, dev = d.rows, d.h, _io_dtype(d), _dev(dy)
    f32, u8 = torch.float32, torch.uint8
    args = [_arg(dy, "dy", N * H, io, dev), _arg(dh_out, "dh_out", N * H, io, dev, True),
            _arg(h, "h", N * H, io, dev), _arg(mask, "mask", N * H, u8, dev, True),
            _arg(mean, "mean", N, f32, dev, True), _arg(rstd, "rstd", N, f32, dev),
            _arg(gamma, "gamma", H, f32, dev), _arg(dx_out, "dx_out", N * H, io, dev, True),
            _arg(dres_out, "dres_out", N * H, io, dev),
            _arg(dgamma_out, "dgamma_out", H, f32, dev),
            _arg(dbeta_out, "dbeta_out", H, f32, dev, True),
            _arg(dbias_out, "dbias_out", H, f32, dev, True)]
    st = lib().sp_region_bwd_noalloc(ctypes.byref(d.c()), *args, _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_region_bwd_noalloc", st)


def sp_region_bwd_exit(d, dh_out, mask, dx_out, dbias_out, workspace, stream=None):
    """Backward of the norm-free exit (forward with gamma = None)."""
    import torch
    N, H, io, dev = d.rows, d.h, _io_dtype(d), _dev(dh_out)
    ws = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().sp_region_bwd_exit(ctypes.byref(d.c()), _arg(dh_out, "dh_out", N * H, io, dev),
                                  _arg(mask, "mask", N * H, torch.uint8, dev, True),
                                  _arg(dx_out, "dx_out", N * H, io, dev),
                                  _arg(dbias_out, "dbias_out", H, torch.float32, dev, True),
                                  ws, ctypes.c_size_t(ws_bytes), _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_region_bwd_exit", st)


def sp_region_bwd_num_launches(d):
    return int(lib().sp_region_bwd_num_launches(ctypes.byref(d.c())))


def sp_region_bwd_launch(d, index, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out,
                         dgamma_out, dbeta_out, dbias_out, workspace, stream=None):
    args = _bwd_args(d, dy, dh_out, h, mask, mean, rstd, gamma, dx_out, dres_out, dgamma_out,
                     dbeta_out, dbias_out, workspace)
    st = lib().sp_region_bwd_launch(ctypes.byref(d.c()), int(index), *args, _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_region_bwd_launch", st)


# ------------------------------------------------------------ ring attention
def sp_ring_attn_workspace_bytes(d):
    return int(lib().sp_ring_attn_workspace_bytes(ctypes.byref(d.c())))


def _ws(workspace):
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(
        workspace.numel() * workspace.element_size())


def sp_ring_attn_fwd(d, q, k, v, o_out, lse_out, workspace, stream=None):
    import torch
    n, dev = d.rows * d.d, _dev(q)
    bf = torch.bfloat16
    st = lib().sp_ring_attn_fwd(ctypes.byref(d.c()), _arg(q, "q", n, bf, dev),
                                _arg(k, "k", d.t * n, bf, dev), _arg(v, "v", d.t * n, bf, dev),
                                _arg(o_out, "o_out", n, bf, dev),
                                _arg(lse_out, "lse_out", d.rows, torch.float32, dev, True),
                                *_ws(workspace), _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_ring_attn_fwd", st)


def sp_ring_attn_fwd_num_launches(d):
    return int(lib().sp_ring_attn_fwd_num_launches(ctypes.byref(d.c())))


def sp_ring_attn_fwd_launch(d, index, q, k, v, o_out, lse_out, workspace, stream=None):
    import torch
    n, dev = d.rows * d.d, _dev(q)
    bf = torch.bfloat16
    st = lib().sp_ring_attn_fwd_launch(ctypes.byref(d.c()), int(index), _arg(q, "q", n, bf, dev),
                                       _arg(k, "k", d.t * n, bf, dev), _arg(v, "v", d.t * n, bf, dev),
                                       _arg(o_out, "o_out", n, bf, dev),
                                       _arg(lse_out, "lse_out", d.rows, torch.float32, dev, True),
                                       *_ws(workspace), _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_ring_attn_fwd_launch", st)


def sp_ring_attn_step(d, step, q, k_blk, v_blk, workspace, stream=None):
    import torch
    n, dev = d.rows * d.d, _dev(q)
    bf = torch.bfloat16
    st = lib().sp_ring_attn_step(ctypes.byref(d.c()), ctypes.c_int32(int(step)),
                                 _arg(q, "q", n, bf, dev), _arg(k_blk, "k_blk", n, bf, dev),
                                 _arg(v_blk, "v_blk", n, bf, dev), *_ws(workspace),
                                 _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_ring_attn_step", st)


def sp_ring_attn_merge(d, o_out, lse_out, workspace, stream=None):
    import torch
    n, dev = d.rows * d.d, _dev(o_out)
    st = lib().sp_ring_attn_merge(ctypes.byref(d.c()), _arg(o_out, "o_out", n, torch.bfloat16, dev),
                                  _arg(lse_out, "lse_out", d.rows, torch.float32, dev, True),
                                  *_ws(workspace), _stream(stream))
    if st != SPR_OK:
        raise SprError("sp_ring_attn_merge", st)


def ring_attn(d, q, k, v, stream=None):
    """Allocates O, lse and the workspace; runs sp_ring_attn_fwd."""
    import torch
    o = torch.empty(d.rows * d.d, dtype=torch.bfloat16, device=q.device)
    lse = torch.empty(d.rows, dtype=torch.float32, device=q.device)
    ws = torch.empty(max(sp_ring_attn_workspace_bytes(d), 256), dtype=torch.uint8, device=q.device)
    sp_ring_attn_fwd(d, q, k, v, o, lse, ws, stream)
    return o, lse


# ------------------------------------------------------------ allocation helpers
def alloc_fwd_outputs(d, device, store_mask=True, norm=True, write_h=True):
    """torch.empty outputs of sp_region_fwd: h, y, mask, mean, rstd.  With
    store_mask=False there is no mask (the backward regenerates it);
    norm=False (the norm-free exit) has no y and statistics; write_h=False
    (only for the norm-only entry) has no h."""
    import torch
    N, H, io = d.rows, d.h, _io_dtype(d)
    e = lambda n, dt: torch.empty(n, dtype=dt, device=device)
    return {"h": e(N * H, io) if write_h else None, "y": e(N * H, io) if norm else None,
            "mask": e(N * H, torch.uint8) if d.p > 0 and store_mask else None,
            "mean": e(N, torch.float32) if norm and d.norm == SPR_LAYERNORM else None,
            "rstd": e(N, torch.float32) if norm else None}


def alloc_bwd_outputs(d, device, want_dbias=True):
    """torch.empty outputs of sp_region_bwd and its workspace (whose contents
    on entry do not matter)."""
    import torch
    N, H, io = d.rows, d.h, _io_dtype(d)
    e = lambda n, dt: torch.empty(n, dtype=dt, device=device)
    ws = max(sp_region_bwd_workspace_bytes(d), 16)
    return {"dx": e(N * H, io), "dres": e(N * H, io), "dgamma": e(H, torch.float32),
            "dbeta": e(H, torch.float32) if d.norm == SPR_LAYERNORM else None,
            "dbias": e(H, torch.float32) if want_dbias else None,
            "workspace": e(ws, torch.uint8)}


def fwd(d, x, bias, residual, gamma, beta, stream=None, store_mask=True, write_h=True):
    """Allocates the outputs and runs sp_region_fwd; returns them as a dict.
    x = None: the norm-only entry; gamma = None: the norm-free exit."""
    o = alloc_fwd_outputs(d, residual.device, store_mask and x is not None, gamma is not None,
                          write_h or x is not None)
    sp_region_fwd(d, x, bias, residual, gamma, beta, o["h"], o["y"], o["mask"], o["mean"],
                  o["rstd"], stream)
    return o


def fwd_rs(d, x_parts, nparts, bias, residual, gamma, beta, stream=None, store_mask=True):
    """Allocates the outputs and runs sp_region_fwd_rs; returns them as a dict."""
    o = alloc_fwd_outputs(d, x_parts.device, store_mask)
    sp_region_fwd_rs(d, x_parts, nparts, bias, residual, gamma, beta, o["h"], o["y"], o["mask"],
                     o["mean"], o["rstd"], stream)
    return o


def bwd(d, dy, dh_out, h, mask, mean, rstd, gamma, want_dbias=True, stream=None):
    """Allocates the outputs and runs sp_region_bwd; returns them as a dict."""
    o = alloc_bwd_outputs(d, dy.device, want_dbias)
    sp_region_bwd(d, dy, dh_out, h, mask, mean, rstd, gamma, o["dx"], o["dres"], o["dgamma"],
                  o["dbeta"], o["dbias"], o["workspace"], stream)
    return o


def _region_function():
    import torch

    class SPRegionFunction(torch.autograd.Function):
        """The region as an autograd function on one shard: (y, h) =
        region(x, residual, bias, gamma, beta).  Inputs are flat [N*h]
        tensors in the I/O type (bias, gamma, beta fp32 [h]; bias and beta
        may be None).  Forward: sp_region_fwd with the mask stored; backward:
        sp_region_bwd from the saved h, mask and statistics, with the gradient
        reaching h from outside the region passed as dh_out."""

        @staticmethod
        def forward(ctx, x, residual, bias, gamma, beta, d):
            o = fwd(d, x, bias, residual, gamma, beta)
            ctx.save_for_backward(o["h"], o["mask"], o["mean"], o["rstd"], gamma)
            ctx.d, ctx.want_dbias = d, bias is not None
            return o["y"], o["h"]

        @staticmethod
        def backward(ctx, dy, dh):
            h, mask, mean, rstd, gamma = ctx.saved_tensors
            if dy is None:
                dy = torch.zeros_like(h)
            g = bwd(ctx.d, dy.contiguous(), None if dh is None else dh.contiguous(), h, mask,
                    mean, rstd, gamma, want_dbias=ctx.want_dbias)
            return g["dx"], g["dres"], g["dbias"], g["dgamma"], g["dbeta"], None

    return SPRegionFunction


def region(d, x, residual, bias, gamma, beta):
    """(y, h) of the region on one shard, differentiable through
    sp_region_bwd (see SPRegionFunction in _region_function)."""
    global _REGION_FN
    if _REGION_FN is None:
        _REGION_FN = _region_function()
    return _REGION_FN.apply(x, residual, bias, gamma, beta, d)


_REGION_FN = None

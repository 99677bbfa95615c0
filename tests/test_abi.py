"""The C ABI on the host: the library loads, exports every function that
include/sp_region.h declares, and rejects invalid calls before any HIP call
(so these run without a GPU).  No compute call is made here."""
import ctypes
import os
import re

import pytest

import dropout_region_amd as spr
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", "sp_region.h"),
           os.path.join(ROOT, "include", "sp_ring_attn.h")]


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(spr.LIB_PATH):
        pytest.fail("libsp_region.so is not built; run __graft_entry__.build()")
    return spr.lib()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sp_(?:region|ring_attn)_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["sp_region_fwd", "sp_region_fwd_rs", "sp_region_bwd",
                            "sp_region_bwd_exit", "sp_region_bwd_noalloc",
                            "sp_region_bwd_workspace_bytes",
                            "sp_region_bwd_num_launches", "sp_region_bwd_launch",
                            "sp_region_activation_bytes", "sp_region_status_string",
                            "sp_ring_attn_workspace_bytes", "sp_ring_attn_fwd",
                            "sp_ring_attn_step", "sp_ring_attn_merge",
                            "sp_ring_attn_fwd_num_launches", "sp_ring_attn_fwd_launch"])


def test_library_exports_every_declared_function(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings(L):
    for st in range(5):
        assert spr.sp_region_status_string(st)
    assert spr.sp_region_status_string(99) == "unknown status"


def _fwd_raw(L, d, ptrs):
    return L.sp_region_fwd(ctypes.byref(d), *[ctypes.c_void_p(p) for p in ptrs], None)


def _good_desc(**kw):
    base = dict(s_local=4, b=2, h=64, shard_index=0, t=1, io=spr.SPR_BF16,
                norm=spr.SPR_LAYERNORM, p=0.1, eps=1e-5, seed=0, offset=0)
    base.update(kw)
    return spr.Desc(**base).c()


# Fake, never-dereferenced device addresses: each call below must fail in the
# host checks, before the library touches HIP.
A = 0x7f0000000000
FWD_OK = [A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x310000, A + 0x400000,
          A + 0x500000, A + 0x600000, A + 0x700000, A + 0x710000]


@pytest.mark.parametrize("field,value,status", [
    ("p", 1.0, spr.SPR_ERR_INVALID_ARG), ("p", -0.5, spr.SPR_ERR_INVALID_ARG),
    ("p", float("nan"), spr.SPR_ERR_INVALID_ARG), ("eps", 0.0, spr.SPR_ERR_INVALID_ARG),
    ("eps", float("inf"), spr.SPR_ERR_INVALID_ARG), ("t", 0, spr.SPR_ERR_INVALID_ARG),
    ("shard_index", 1, spr.SPR_ERR_INVALID_ARG), ("shard_index", -1, spr.SPR_ERR_INVALID_ARG),
    ("h", 0, spr.SPR_ERR_INVALID_ARG), ("s_local", 0, spr.SPR_ERR_INVALID_ARG),
    ("io", 5, spr.SPR_ERR_INVALID_ARG), ("norm", 2, spr.SPR_ERR_INVALID_ARG),
    ("h", 60, spr.SPR_ERR_UNSUPPORTED), ("h", 32776, spr.SPR_ERR_UNSUPPORTED),
    ("fwd_kernel", 3, spr.SPR_ERR_INVALID_ARG), ("fwd_kernel", -1, spr.SPR_ERR_INVALID_ARG),
    ("bwd_path", 3, spr.SPR_ERR_INVALID_ARG), ("bwd_tile_rows", 8, spr.SPR_ERR_INVALID_ARG),
    ("bwd_tile_rows", 40, spr.SPR_ERR_INVALID_ARG),
    ("bwd_tile_rows", 2 ** 21, spr.SPR_ERR_INVALID_ARG),
])
def test_fwd_rejects_bad_desc(L, field, value, status):
    d = _good_desc(**{field: value})
    assert _fwd_raw(L, d, FWD_OK) == status


def test_launch_choices_are_checked_by_every_entry_point(L):
    """A nonzero reserved word, or a launch choice out of range, is an
    invalid descriptor for the backward and its workspace query too."""
    for bad in (dict(bwd_path=-2), dict(bwd_tile_rows=24)):
        d = _good_desc(**bad)
        assert L.sp_region_bwd_workspace_bytes(ctypes.byref(d)) == 0, bad
        assert L.sp_region_bwd_num_launches(ctypes.byref(d)) == 0, bad
    d = _good_desc()
    d.reserved = 1
    assert _fwd_raw(L, d, FWD_OK) == spr.SPR_ERR_INVALID_ARG
    assert L.sp_region_bwd_workspace_bytes(ctypes.byref(d)) == 0
    for ok in (dict(fwd_kernel=spr.SPR_FWD_STREAM), dict(bwd_path=spr.SPR_BWD_SPLIT),
               dict(bwd_tile_rows=48)):
        assert L.sp_region_bwd_workspace_bytes(ctypes.byref(_good_desc(**ok))) > 0, ok


def _fwd_rs_raw(L, d, nparts, ptrs):
    return L.sp_region_fwd_rs(ctypes.byref(d), ctypes.c_void_p(ptrs[0]), ctypes.c_int32(nparts),
                              *[ctypes.c_void_p(p) for p in ptrs[1:]], None)


def test_fwd_rs_checks(L):
    d = _good_desc()                             # N*h*2 = 1 KiB per slab
    assert _fwd_rs_raw(L, d, 0, FWD_OK) == spr.SPR_ERR_INVALID_ARG
    assert _fwd_rs_raw(L, d, -3, FWD_OK) == spr.SPR_ERR_INVALID_ARG
    assert _fwd_rs_raw(L, d, 1025, FWD_OK) == spr.SPR_ERR_INVALID_ARG
    bad = list(FWD_OK)
    bad[5] = FWD_OK[0] + 3 * 1024                # h_out inside slab 3 of 4
    assert _fwd_rs_raw(L, d, 4, bad) == spr.SPR_ERR_INVALID_ARG
    assert _fwd_rs_raw(L, _good_desc(h=60), 4, FWD_OK) == spr.SPR_ERR_UNSUPPORTED


def test_variant_rules(L):
    d0 = _good_desc(p=0.0)
    entry = list(FWD_OK)
    entry[0] = 0                                 # no x ...
    assert _fwd_raw(L, _good_desc(), entry, ) == spr.SPR_ERR_INVALID_ARG   # ... with p > 0
    assert _fwd_raw(L, d0, entry) == spr.SPR_ERR_INVALID_ARG              # ... with a bias
    both = list(entry)
    both[1] = 0
    both[3] = 0                                  # neither x nor gamma
    assert _fwd_raw(L, d0, both) == spr.SPR_ERR_INVALID_ARG
    exit_ = list(FWD_OK)
    exit_[3] = 0                                 # no gamma, but y/beta/mean/rstd given
    assert _fwd_raw(L, d0, exit_) == spr.SPR_ERR_INVALID_ARG
    exit_[4] = exit_[6] = exit_[8] = 0
    assert _fwd_raw(L, d0, exit_) == spr.SPR_ERR_INVALID_ARG              # rstd still given
    exit_[5] = 0
    exit_[9] = 0                                 # ... and no h_out
    assert _fwd_raw(L, d0, exit_) == spr.SPR_ERR_INVALID_ARG
    call = lambda dho, dx, ws, n: L.sp_region_bwd_exit(
        ctypes.byref(d0), ctypes.c_void_p(dho), None, ctypes.c_void_p(dx),
        ctypes.c_void_p(A + 0x300000), ctypes.c_void_p(ws), ctypes.c_size_t(n), None)
    assert call(0, A + 0x100000, A + 0x200000, 1 << 20) == spr.SPR_ERR_INVALID_ARG  # no dh_out
    assert call(A, 0, A + 0x200000, 1 << 20) == spr.SPR_ERR_INVALID_ARG            # no dx_out
    assert call(A, A + 0x100000, 0, 0) == spr.SPR_ERR_WORKSPACE                    # dbias, no ws
    assert call(A, A, A + 0x200000, 1 << 20) == spr.SPR_ERR_INVALID_ARG            # dx aliases


def test_fwd_pointer_rules(L):
    d = _good_desc()
    bad = list(FWD_OK)
    bad[0] = 0                                   # x missing
    assert _fwd_raw(L, d, bad) == spr.SPR_ERR_INVALID_ARG
    bad = list(FWD_OK)
    bad[0] = A + 8                               # x misaligned
    assert _fwd_raw(L, d, bad) == spr.SPR_ERR_INVALID_ARG
    bad = list(FWD_OK)
    bad[7] = A + 0x600004                        # mask misaligned (8-byte words)
    assert _fwd_raw(L, d, bad) == spr.SPR_ERR_INVALID_ARG
    bad = list(FWD_OK)
    bad[9] = 0                                   # rstd missing
    assert _fwd_raw(L, d, bad) == spr.SPR_ERR_INVALID_ARG
    bad = list(FWD_OK)
    bad[4] = 0                                   # beta missing for LayerNorm
    assert _fwd_raw(L, d, bad) == spr.SPR_ERR_INVALID_ARG
    rms = _good_desc(norm=spr.SPR_RMSNORM)
    assert _fwd_raw(L, rms, FWD_OK) == spr.SPR_ERR_INVALID_ARG   # beta given for RMSNorm
    bad = list(FWD_OK)
    bad[5] = FWD_OK[0] + 16                      # h_out overlaps x
    assert _fwd_raw(L, d, bad) == spr.SPR_ERR_INVALID_ARG
    bad = list(FWD_OK)
    bad[6] = FWD_OK[5]                           # y_out aliases h_out
    assert _fwd_raw(L, d, bad) == spr.SPR_ERR_INVALID_ARG


def test_bwd_launch_count(L):
    assert L.sp_region_bwd_num_launches(ctypes.byref(_good_desc())) == 2         # fused
    assert L.sp_region_bwd_num_launches(ctypes.byref(_good_desc(h=25600))) == 3  # split
    assert L.sp_region_bwd_num_launches(ctypes.byref(_good_desc(p=1.0))) == 0


def test_bwd_launch_index_checked(L):
    d = _good_desc()
    need = L.sp_region_bwd_workspace_bytes(ctypes.byref(d))
    ptrs = [A + i * 0x100000 for i in range(12)]
    ptrs[1] = 0
    for index in (-1, 2, 7):
        assert L.sp_region_bwd_launch(ctypes.byref(d), index, *[ctypes.c_void_p(p) for p in ptrs],
                                      ctypes.c_void_p(A + 0x4000000), ctypes.c_size_t(need),
                                      None) == spr.SPR_ERR_INVALID_ARG


def test_bwd_workspace_rules(L):
    d = _good_desc()
    need = L.sp_region_bwd_workspace_bytes(ctypes.byref(d))
    assert need > 0 and need % 256 == 0
    assert L.sp_region_bwd_workspace_bytes(ctypes.byref(_good_desc(p=2.0))) == 0
    ptrs = [A + i * 0x100000 for i in range(12)]
    ptrs[1] = 0                                  # no dh_out
    call = lambda ws, n: L.sp_region_bwd(ctypes.byref(d), *[ctypes.c_void_p(p) for p in ptrs],
                                         ctypes.c_void_p(ws), ctypes.c_size_t(n), None)
    assert call(0, need) == spr.SPR_ERR_WORKSPACE
    assert call(A + 0x4000000, need - 1) == spr.SPR_ERR_WORKSPACE
    d_rms = _good_desc(norm=spr.SPR_RMSNORM)     # dbeta given for RMSNorm
    assert L.sp_region_bwd(ctypes.byref(d_rms), *[ctypes.c_void_p(p) for p in ptrs],
                           ctypes.c_void_p(A + 0x4000000), ctypes.c_size_t(need),
                           None) == spr.SPR_ERR_INVALID_ARG


@pytest.mark.parametrize("io,norm,p", [(spr.SPR_BF16, spr.SPR_LAYERNORM, 0.1),
                                       (spr.SPR_F32, spr.SPR_LAYERNORM, 0.1),
                                       (spr.SPR_BF16, spr.SPR_RMSNORM, 0.0),
                                       (spr.SPR_F32, spr.SPR_RMSNORM, 0.3)])
def test_activation_bytes_agree_with_oracle(L, olib, io, norm, p):
    for (s_local, b, h) in [(256, 4, 6144), (256, 8, 12288), (4096, 1, 8192), (2048, 4, 25600),
                            (64, 2, 256)]:
        d = spr.Desc(s_local=s_local, b=b, h=h, io=io, norm=norm, p=p)
        od = oracle.Desc(s_local=s_local, b=b, h=h, io=io, norm=norm, p=p)
        assert spr.sp_region_activation_bytes(d) == oracle.activation_bytes(od, L=olib)


def test_ring_attn_rejects_bad_calls(L):
    def desc(**kw):
        base = dict(s_local=128, b=1, heads=2, d=128, t=4, rank=1, scale=0.0)
        base.update(kw)
        return spr.AttnDesc(**base).c()
    assert L.sp_ring_attn_workspace_bytes(ctypes.byref(desc())) > 0
    for bad in (dict(d=96), dict(rank=4), dict(rank=-1), dict(t=0), dict(s_local=0),
                dict(heads=70000), dict(scale=float("nan")), dict(scale=-1.0),
                dict(steps_per_wg=3), dict(steps_per_wg=8), dict(steps_per_wg=-1)):
        d = desc(**bad)
        assert L.sp_ring_attn_workspace_bytes(ctypes.byref(d)) == 0, bad
        assert L.sp_ring_attn_fwd(ctypes.byref(d), *[ctypes.c_void_p(A + i * 0x1000000) for i in range(5)],
                                  ctypes.c_void_p(A + 0x8000000), ctypes.c_size_t(1 << 30),
                                  None) == spr.SPR_ERR_INVALID_ARG, bad
    d = desc()
    need = L.sp_ring_attn_workspace_bytes(ctypes.byref(d))
    ptrs = [ctypes.c_void_p(A + i * 0x1000000) for i in range(5)]
    assert L.sp_ring_attn_fwd(ctypes.byref(d), *ptrs, ctypes.c_void_p(A + 0x8000000),
                              ctypes.c_size_t(need - 1), None) == spr.SPR_ERR_WORKSPACE
    ptrs[3] = ctypes.c_void_p(A + 0x1000000)     # o_out aliases k
    assert L.sp_ring_attn_fwd(ctypes.byref(d), *ptrs, ctypes.c_void_p(A + 0x8000000),
                              ctypes.c_size_t(need), None) == spr.SPR_ERR_INVALID_ARG
    for step in (-1, 4):
        assert L.sp_ring_attn_step(ctypes.byref(d), step, *[ctypes.c_void_p(A + i * 0x1000000)
                                                           for i in range(3)],
                                   ctypes.c_void_p(A + 0x8000000), ctypes.c_size_t(need),
                                   None) == spr.SPR_ERR_INVALID_ARG


def test_ring_attn_launch_count_and_index(L):
    """The fused forward is two launches; an index outside them, or a bad
    desc, is rejected before anything is launched."""
    def desc(**kw):
        base = dict(s_local=128, b=1, heads=2, d=128, t=4, rank=1, scale=0.0)
        base.update(kw)
        return spr.AttnDesc(**base).c()
    d = desc()
    assert L.sp_ring_attn_fwd_num_launches(ctypes.byref(d)) == 2
    assert L.sp_ring_attn_fwd_num_launches(ctypes.byref(desc(d=96))) == 0
    need = L.sp_ring_attn_workspace_bytes(ctypes.byref(d))
    ptrs = [ctypes.c_void_p(A + i * 0x1000000) for i in range(5)]
    for index in (-1, 2):
        assert L.sp_ring_attn_fwd_launch(ctypes.byref(d), index, *ptrs,
                                         ctypes.c_void_p(A + 0x8000000), ctypes.c_size_t(need),
                                         None) == spr.SPR_ERR_INVALID_ARG, index
    assert L.sp_ring_attn_fwd_launch(ctypes.byref(desc(rank=4)), 0, *ptrs,
                                     ctypes.c_void_p(A + 0x8000000), ctypes.c_size_t(need),
                                     None) == spr.SPR_ERR_INVALID_ARG
    assert L.sp_ring_attn_fwd_launch(ctypes.byref(d), 0, *ptrs, ctypes.c_void_p(A + 0x8000000),
                                     ctypes.c_size_t(need - 1), None) == spr.SPR_ERR_WORKSPACE


def test_activation_bytes_count_the_buffers_a_forward_keeps(L):
    """The bytes of the buffers a forward call writes and keeps (h, mask,
    statistics for the backward; y for the next block), as allocated for the
    call, equal sp_region_activation_bytes; two calls per layer give the
    replicated band divided by t, 10*s*b*h/t bytes plus the statistics."""
    import torch
    from sp_inputs import WORKLOADS
    for name, w in WORKLOADS.items():
        d = spr.Desc(s_local=w.s_local, b=w.b, h=w.h, t=w.t, io=w.io, norm=w.norm, p=w.p,
                     eps=w.eps)
        o = spr.alloc_fwd_outputs(d, torch.device("meta"))
        nbytes = lambda k: 0 if o[k] is None else o[k].numel() * o[k].element_size()
        saved = nbytes("h") + nbytes("mask") + nbytes("mean") + nbytes("rstd")
        assert spr.sp_region_activation_bytes(d) == (saved, nbytes("y")), name
        if name.startswith("1t_"):
            stats = 2 * 8 * w.rows
            assert 2 * (saved + nbytes("y")) - stats == 10 * w.s * w.b * w.h // w.t, name
        free = spr.alloc_fwd_outputs(d, torch.device("meta"), store_mask=False)
        kept = sum(0 if free[k] is None else free[k].numel() * free[k].element_size()
                   for k in ("h", "mask", "mean", "rstd"))
        assert saved - kept == (w.rows * w.h if w.p > 0 else 0), name


def test_noalloc_backward_checks(L):
    """The allocation-free backward checks its arguments like sp_region_bwd,
    and a shard whose scratch need exceeds the fixed array is
    SPR_ERR_WORKSPACE -- all on the host, before anything is launched."""
    G = 1 << 32                                  # fake buffers 4 GiB apart

    def call(d, dy=A):
        ptrs = [dy, 0, A + 2 * G, A + 3 * G, A + 4 * G, A + 5 * G, A + 6 * G, A + 7 * G,
                A + 8 * G, A + 9 * G, A + 10 * G, A + 11 * G]
        return L.sp_region_bwd_noalloc(ctypes.byref(d), *[ctypes.c_void_p(p) for p in ptrs],
                                       None)
    assert call(_good_desc(p=2.0)) == spr.SPR_ERR_INVALID_ARG
    assert call(_good_desc(), dy=0) == spr.SPR_ERR_INVALID_ARG
    big = _good_desc(s_local=2048, b=4, h=25600)
    assert L.sp_region_bwd_workspace_bytes(ctypes.byref(big)) > 64 << 20
    assert call(big) == spr.SPR_ERR_WORKSPACE

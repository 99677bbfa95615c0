"""Pins of the activation accounting against the pages' printed figures.

Fixture: tests/golden/sp_math_worked_example.json ("Sequence parallel math",
section "A worked numeric example", and the replicated-band breakdown of
section "What tensor parallelism leaves replicated").
"""
import json
import os

import numpy as np
import pytest

import oracle
from sp_inputs import WORKLOADS

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "sp_math_worked_example.json")))


def test_worked_example_figures(olib):
    sh, pr = GOLD["shape"], GOLD["printed"]
    s, b, h, a, t = sh["s"], sh["b"], sh["h"], sh["a"], sh["t"]
    full, tp, tp_sp = oracle.layer_activation_elems(s, b, h, a, t, L=olib)
    sbh = s * b * h
    assert 5 * a * s / h == pr["five_a_s_over_h"]
    assert abs(sbh - pr["sbh_elements"]) / pr["sbh_elements"] < 5e-4
    assert tp / sbh == pr["tp_only_coefficient"]
    assert tp_sp / sbh == pr["tp_sp_coefficient"]
    assert full / t == tp_sp                       # the ideal 1/t scaling
    gb = lambda e: e * pr["bytes_per_element_fp16"] / 1e9
    assert round(gb(tp), 2) == pr["tp_only_gb_per_layer_device"]
    assert round(gb(tp_sp), 2) == pr["tp_sp_gb_per_layer_device"]
    assert round(100 * (1 - tp_sp / tp)) == pr["reduction_percent"]
    assert round(gb(tp - tp_sp), 2) == pr["saved_gb_per_layer_device"]
    assert abs(gb(tp - tp_sp) * pr["layers"] - pr["saved_gb_stack_order_of"]) < 5
    # the gap between TP and TP+SP is the replicated band: 10*sbh - 10*sbh/t
    k = GOLD["replicated_band"]["coefficient"]
    assert tp - tp_sp == pytest.approx(k * sbh - k * sbh / t, rel=1e-12)


def test_region_bytes_reproduce_replicated_band(olib):
    """Two region calls per layer (pre-attention, pre-MLP), bf16 with a
    one-byte mask, keep exactly 10*s*b*h/t bytes of h, masks and block
    inputs, plus the fp32 per-token statistics."""
    k = GOLD["replicated_band"]["coefficient"]
    for t in (1, 2, 4, 8):
        w = WORKLOADS[f"1t_h25600_t{t}"]
        d = oracle.Desc(s_local=w.s_local, b=w.b, h=w.h, t=w.t, io=w.io, norm=w.norm, p=w.p,
                        eps=w.eps)
        saved, retained = oracle.activation_bytes(d, L=olib)
        per_layer = 2 * (saved + retained)
        stats = 2 * 8 * w.rows
        assert per_layer - stats == k * w.s * w.b * w.h // t
    # RMSNorm keeps one statistic per token; p = 0 keeps no mask
    d = oracle.Desc(s_local=4096, b=1, h=8192, io=oracle.BF16, norm=oracle.RMSNORM, p=0.0,
                    eps=1e-6)
    saved, retained = oracle.activation_bytes(d, L=olib)
    assert saved == 4096 * 8192 * 2 + 4096 * 4 and retained == 4096 * 8192 * 2

"""The benchmark's algorithmic byte and FLOP counts, from the element sizes
(no GPU).  Forward: read x and residual, write h and y (2 bytes each for
bf16, 4 for fp32), one mask byte per element when p > 0, bias/gamma/beta
read once per call, fp32 statistics per row.  Backward: read dy and h, the
mask, write dx and dresidual, read gamma and the statistics, write the three
parameter gradients."""
import pytest

import bench
from sp_inputs import ATTN_WORKLOADS, WORKLOADS


@pytest.mark.parametrize("name,fwd,bwd", [
    # 22B: [256, 4, 6144] bf16 LayerNorm p = 0.1
    ("22b_h6144_t8", 6291456 * 9 + 3 * 6144 * 4 + 2 * 1024 * 4,
     6291456 * 9 + 2 * 1024 * 4 + 6144 * 4 + 3 * 6144 * 4),
    # 175B: [256, 8, 12288], one call
    ("175b_h12288_t8", 25165824 * 9 + 3 * 12288 * 4 + 2 * 2048 * 4,
     25165824 * 9 + 2 * 2048 * 4 + 12288 * 4 + 3 * 12288 * 4),
    # long-sequence RMSNorm [4096, 1, 8192]: no beta, one statistic
    ("longseq_rms_h8192_t8_p0.1", 33554432 * 9 + 2 * 8192 * 4 + 4096 * 4,
     33554432 * 9 + 4096 * 4 + 8192 * 4 + 2 * 8192 * 4),
    ("longseq_rms_h8192_t8_p0", 33554432 * 8 + 2 * 8192 * 4 + 4096 * 4,
     33554432 * 8 + 4096 * 4 + 8192 * 4 + 2 * 8192 * 4),
    # tiny fp32 [64, 2, 256]: 4 bytes per element
    ("tiny_fp32_t2", 32768 * 17 + 3 * 256 * 4 + 2 * 128 * 4,
     32768 * 17 + 2 * 128 * 4 + 256 * 4 + 3 * 256 * 4),
])
def test_region_bytes(name, fwd, bwd):
    f, r, g = bench.algorithmic_bytes(WORKLOADS[name])
    assert f == fwd and r + g == bwd


def test_region_byte_variants():
    w = WORKLOADS["22b_h6144_t8"]
    E, H, N = w.elems, w.h, w.rows
    f, r, g = bench.algorithmic_bytes(w, with_dh_out=True)
    assert r == E * 11 + 2 * N * 4 + H * 4                 # dh_out read too
    f, r, g = bench.algorithmic_bytes(w, mask_stored=False)
    assert f == E * 8 + 3 * H * 4 + 2 * N * 4               # no mask written or read
    f, r, g = bench.algorithmic_bytes(w, x_parts=8)
    assert f == E * ((8 + 3) * 2 + 1) + 3 * H * 4 + 2 * N * 4   # eight slabs of x read
    fe, be = bench.variant_bytes(w, "entry")
    assert fe == E * 4 + 2 * H * 4 + 2 * N * 4              # residual in, y out
    fx, bx = bench.variant_bytes(w, "exit")
    assert fx == E * 7 + H * 4 and bx == E * 5 + H * 4      # x, res in, h, mask out / dh, mask in, dx out


def test_attention_flops():
    w = ATTN_WORKLOADS["ring_attn_s32k_t8_h8192"]
    assert w.s_local == 4096
    # Q K^T and P V over 32768 keys: 2 * 2 * 4096 * 32768 * 128 per head, 8 heads
    assert w.flops == 4 * 4096 * 32768 * 128 * 8 == 549755813888


def test_more_than_one_gpu_is_refused():
    """bench.py runs on one GPU: --gpus N > 1 exits with status 2 and says so
    (before anything touches a GPU)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _pmc_csv(path, rows):
    import csv
    import os
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_counters_summary_merges_passes(tmp_path, monkeypatch):
    """Two --pmc passes (different counters) go into one table, each counter
    averaged over its dispatches; kernels outside the library are left out."""
    step = "spr::ring_attn_step_kernel<128, true>(spr::AttnArgs)"
    _pmc_csv(str(tmp_path / "p1"), [(1, step, "SQ_WAVES", 10), (2, step, "SQ_WAVES", 30),
                                    (3, "elementwise_kernel", "SQ_WAVES", 99)])
    _pmc_csv(str(tmp_path / "p2"), [(1, step, "SQ_LDS_BANK_CONFLICT", 4), (2, step, "SQ_LDS_BANK_CONFLICT", 8)])
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    bench.counters_summary([str(tmp_path / "p1"), str(tmp_path / "p2")], "ring_attn_s2k_t8_d128", "cmd")
    text = (tmp_path / "ring_attn_s2k_t8_d128_counters.md").read_text()
    assert "## ring_attn_step_kernel" in text
    assert "| SQ_WAVES | 20 |" in text
    assert "| SQ_LDS_BANK_CONFLICT | 6 |" in text
    assert "elementwise" not in text

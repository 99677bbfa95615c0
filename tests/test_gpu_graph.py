"""HIP graph capture of the region: the library's launches, recorded in a
graph on a capture stream and replayed, give the eager results bit for bit
on every replay, with eager work (the outputs cleared) between replays.
The library records no memset and allocates nothing, so its launches are
safe to capture; this checks it."""
import numpy as np
import pytest

import dropout_region_amd as spr
from sp_inputs import make_inputs
from tests import parity as P

pytestmark = pytest.mark.gpu


def _outputs(d, dev):
    o = spr.alloc_fwd_outputs(d, dev)
    o.update({"b_" + k: v for k, v in spr.alloc_bwd_outputs(d, dev).items()})
    return o


def _run(d, a, o):
    spr.sp_region_fwd(d, a["x"], a["bias"], a["res"], a["gamma"], a["beta"], o["h"], o["y"],
                      o["mask"], o["mean"], o["rstd"])
    spr.sp_region_bwd(d, a["dy"], a["dh_out"], o["h"], o["mask"], o["mean"], o["rstd"],
                      a["gamma"], o["b_dx"], o["b_dres"], o["b_dgamma"], o["b_dbeta"],
                      o["b_dbias"], o["b_workspace"])


_KEYS = ("h", "y", "mask", "mean", "rstd", "b_dx", "b_dres", "b_dgamma", "b_dbeta", "b_dbias")


@pytest.mark.parametrize("h,rows,fwd_path,bwd_path", [(6144, 64, "rows", "fused"),
                                                      (6144, 64, "rows", "split"),
                                                      (8192, 1200, "stream", None),
                                                      (25600, 6, None, None)])
def test_graph_replays_equal_eager(h, rows, fwd_path, bwd_path):
    import torch
    dev = torch.device("cuda:0")
    d = spr.Desc(s_local=rows, b=1, h=h, shard_index=1, t=2, p=0.1)
    print(f"[case] graph h={h} rows={rows} fwd={fwd_path} bwd={bwd_path}", flush=True)
    inp = make_inputs(d.rows, h, d.io, seed=5, dh_out=True)
    a = {"x": P.to_device(inp["x"], d.io), "res": P.to_device(inp["residual"], d.io),
         "dy": P.to_device(inp["dy"], d.io), "dh_out": P.to_device(inp["dh_out"], d.io),
         "bias": P.to_device(inp["bias"]), "gamma": P.to_device(inp["gamma"]),
         "beta": P.to_device(inp["beta"])}
    d = P.tuned(d, fwd=fwd_path, bwd=bwd_path)
    eager = _outputs(d, dev)
    _run(d, a, eager)
    torch.cuda.synchronize()
    want = {k: P.to_host(eager[k]) for k in _KEYS}

    o = _outputs(d, dev)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        _run(d, a, o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in _KEYS:
            o[k].zero_()
        _run(d, a, eager)                    # eager launches between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in _KEYS:
            got = P.to_host(o[k])
            assert np.array_equal(np.asarray(got).view(np.uint8), np.asarray(want[k]).view(np.uint8)), \
                f"replay {rep}: {k} differs from the eager result"


def test_concurrent_calls_on_two_streams_equal_serial():
    """The library keeps no state between calls: two region calls (different
    shapes, shards and paths' plans, separate outputs and workspaces) issued
    on two streams at once, many times over, give the serial results bit for
    bit."""
    import torch
    dev = torch.device("cuda:0")
    cases = [(spr.Desc(s_local=96, b=2, h=6144, shard_index=3, t=4, p=0.1), 21),
             (spr.Desc(s_local=40, b=1, h=25600, shard_index=0, t=2, p=0.2), 22)]
    print("[case] concurrent region calls on two streams", flush=True)
    runs = []
    for d, seed in cases:
        inp = make_inputs(d.rows, d.h, d.io, seed=seed, dh_out=True)
        a = {"x": P.to_device(inp["x"], d.io), "res": P.to_device(inp["residual"], d.io),
             "dy": P.to_device(inp["dy"], d.io), "dh_out": P.to_device(inp["dh_out"], d.io),
             "bias": P.to_device(inp["bias"]), "gamma": P.to_device(inp["gamma"]),
             "beta": P.to_device(inp["beta"])}
        serial = _outputs(d, dev)
        _run(d, a, serial)
        torch.cuda.synchronize()
        runs.append((d, a, {k: P.to_host(serial[k]) for k in _KEYS}, _outputs(d, dev)))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(20):
        for (d, a, _, o), s in zip(runs, streams):
            with torch.cuda.stream(s):
                _run(d, a, o)
    torch.cuda.synchronize()
    for d, _, want, o in runs:
        for k in _KEYS:
            got = P.to_host(o[k])
            assert np.array_equal(np.asarray(got).view(np.uint8),
                                  np.asarray(want[k]).view(np.uint8)), f"h={d.h}: {k} differs"

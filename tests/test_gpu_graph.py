"""The hot path captured into a HIP graph: every replay equals the eager result.

The binding launches on torch's current stream, so capture works through the
C ABI unchanged.  Replays are interleaved with eager work and synchronisation
and each one is compared with the eager outputs (bit-exact: same kernels,
same inputs)."""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import doge_dynamic_mask_amd as dma
    wl = si.Workload("g", "bf16", 2, 8, 4, 700, 128, 256, pad_lo=400, pad_hi=700, seed=91)
    inp = si.make_inputs(wl)
    Q, K, V = to_dev(inp["Q"]), to_dev(inp["K"]), to_dev(inp["V"])
    W, A, bias, seq = to_dev(inp["W"]), to_dev(inp["A"]), to_dev(inp["bias"]), to_dev(inp["seqlens"])
    dt = torch.empty((wl.B, wl.Hkv, wl.S), dtype=torch.float32, device="cuda:0")
    tau, tie = torch.empty_like(dt), torch.empty(dt.shape, dtype=torch.int32, device="cuda:0")
    O = torch.empty_like(Q)
    lens = seq
    q = torch.stack([Q[b, int(inp["seqlens"][b]) - 1] for b in range(wl.B)]).contiguous()
    out = torch.empty_like(q)
    kept = torch.empty((wl.B, wl.Hkv, wl.w), dtype=torch.int32, device="cuda:0")
    ws = torch.empty(dma.decode_workspace_bytes(wl.B, wl.S, wl.Hq, wl.Hkv, wl.d, wl.w), dtype=torch.uint8,
                     device="cuda:0")

    def run():
        dma.dt(V, W, A, bias, out=dt)
        dma.select(dt, wl.w, seq, tau=tau, tie=tie)
        dma.attn_fwd(Q, K, V, dt, tau, tie, wl.w, seq, out=O)
        o2, k2 = dma.decode(q, K, V, dt, lens, wl.w, kept=True, out=out, workspace=ws)
        kept.copy_(k2)

    run()
    torch.cuda.synchronize()
    ref = [to_host(t).copy() for t in (dt, tau, tie, O, out, kept)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for t in (dt, tau, O, out):
            t.zero_()
        torch.cuda.synchronize()
        _ = (Q.float() * 2).sum()  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = [to_host(t) for t in (dt, tau, tie, O, out, kept)]
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b)

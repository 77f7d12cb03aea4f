"""GPU parity of the sliding-window variant: dma_select_window (bit-exact) and
dma_attn_window_fwd (2e-2 abs, bf16) against the oracle with the same window.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dma():
    import doge_dynamic_mask_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


SEL_CASES = [
    # B, Hkv, S, w, win, kind, padded
    (1, 1, 1, 1, 1, "lognormal", False),
    (2, 2, 100, 7, 5, "lognormal", True),       # win < w: canonical pairs only
    (2, 2, 100, 7, 30, "dyadic", True),
    (1, 3, 700, 64, 256, "few", False),
    (1, 2, 700, 1, 64, "lognormal", False),     # w = 1: the window's running argmax
    (2, 1, 3000, 300, 1000, "wide", True),
    (1, 2, 3000, 300, 3003, "const", False),    # window wider than the sequence
    (1, 1, 5000, 2048, 4096, "lognormal", False),
    # windows of at least 64 go through the chunked band selector: windows
    # just above a chunk, w close to the window, ties, padding, both chunk sizes
    (1, 1, 4500, 30, 100, "lognormal", True),
    (1, 2, 900, 120, 130, "dyadic", True),
    (2, 2, 5000, 500, 700, "few", True),
    (1, 1, 4200, 127, 128, "const", False),
    # windows longer than the selector stages in LDS (8192 keys): the common
    # range is binned by a sample of its keys; rows 9001 long, so the second
    # row is not 16-byte aligned
    (1, 2, 9001, 1000, 8700, "spiky", False),
]


@pytest.mark.parametrize("B,Hkv,S,w,win,kind,padded", SEL_CASES)
def test_select_window_bit_exact(dma, oracle_mod, B, Hkv, S, w, win, kind, padded):
    dt = si.make_dt((B, Hkv, S), kind, seed=S + w + win)
    seq = si.make_lengths(B, 1, S, seed=win) if padded else None
    tau, tie = dma.select_window(to_dev(dt), w, win, to_dev(seq))
    rt, ri = oracle_mod.select(dt, w, seq, win=win)
    np.testing.assert_array_equal(to_host(tie), ri)
    np.testing.assert_array_equal(to_host(tau), rt)


ATTN_CASES = [
    # B, S, Hq, Hkv, d, w, win, kind, lens
    (2, 200, 4, 2, 64, 20, 50, "lognormal", (200, 120)),
    (1, 300, 8, 1, 128, 64, 16, "dyadic", None),        # win < w
    (2, 257, 2, 2, 64, 33, 100, "few", None),
    (1, 190, 1, 1, 64, 7, 190, "const", None),
    (2, 97, 16, 2, 128, 10, 40, "lognormal", (97, 1)),
    (1, 2600, 4, 2, 64, 300, 1500, "lognormal", None),   # candidate lists over several scan steps
    # wider windows than the attention kernel's LDS list holds: the window range is walked
    (1, 4700, 2, 1, 64, 4000, 4500, "wide", None),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,d,w,win,kind,lens", ATTN_CASES)
def test_attn_window_elementwise(dma, oracle_mod, B, S, Hq, Hkv, d, w, win, kind, lens):
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", S + win)
    dt = si.make_dt((B, Hkv, S), kind, S + 1)
    seq = None if lens is None else np.array(lens, np.int32)
    dtd, sd = to_dev(dt), to_dev(seq)
    tau, tie = dma.select_window(dtd, w, win, sd)
    O = dma.attn_window_fwd(to_dev(Q), to_dev(K), to_dev(V), dtd, tau, tie, w, win, sd)
    torch.cuda.synchronize()
    ref = oracle_mod.attn(Q, K, V, dt, w, seq, win=win)
    err = np.abs(to_host(O).astype(np.float64) - ref)
    assert err.max() <= 2e-2, err.max()


def test_window_full_size_long_sampled(dma, oracle_mod):
    """The long workload (B1 Hq16 Hkv8 S8192 d128 w2048) under a 4096-position
    window: every row's threshold pair exact, sampled rows' outputs."""
    wl = si.WORKLOADS["long"]
    win = 4096
    inp = si.make_inputs(wl)
    dt = oracle_mod.dt(inp["V"], inp["W"], inp["bias"], inp["A"]).astype(np.float32)
    dtd = to_dev(dt)
    tau, tie = dma.select_window(dtd, wl.w, win)
    O = dma.attn_window_fwd(to_dev(inp["Q"]), to_dev(inp["K"]), to_dev(inp["V"]), dtd, tau, tie, wl.w, win)
    torch.cuda.synchronize()
    rt, ri = oracle_mod.select(dt, wl.w, win=win)
    np.testing.assert_array_equal(to_host(tie), ri)
    np.testing.assert_array_equal(to_host(tau), rt)
    rng = np.random.default_rng(5)
    rows = [(0, g, i) for g in (0, wl.Hkv - 1) for i in (0, 1, 2047, 2048, 4095, 4096, 4097, 8191)]
    rows += [(0, int(rng.integers(wl.Hkv)), int(rng.integers(wl.S))) for _ in range(48)]
    rows = np.array(rows, np.int32)
    ref = oracle_mod.attn(inp["Q"], inp["K"], inp["V"], dt, wl.w, rows=rows, win=win)
    got = to_host(O)
    G = wl.Hq // wl.Hkv
    for n, (b, g, i) in enumerate(rows):
        assert np.abs(got[b, i, g * G:(g + 1) * G] - ref[n]).max() <= 2e-2, (b, g, i)

"""GPU parity of the backward: dma_attn_bwd and dma_dt_bwd against the fp64
oracle (oracle.attn_bwd, oracle.dt_bwd) on the same seeded inputs.

Bars.  dQ, dK, dV come from matrix-core products whose operands p and ds are
rounded to bf16 (relative rounding 2^-9 each) and are stored in bf16; the
terms of a gradient partly cancel (sum_j ds_ij = 0 for every row), so the
error is measured against the largest entry of the gradient:
|gpu - oracle| <= 2e-2 max|oracle| (observed below 1e-2).  ddt is summed in
float32 from unrounded weights: 1e-3 max|oracle|.  dt_bwd is float32 from
end to end: dW, dbias, dA within 1e-4 max|oracle|; the value gradient is
added in place to a bf16 array, so it is compared with half a bf16 ulp of
the sum plus 1e-4 max|oracle|.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.gpu_util import host_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dma():
    import doge_dynamic_mask_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def _rel_check(name, got, ref, bound):
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float(np.abs(got.astype(np.float64) - ref).max())
    assert err <= bound * scale, f"{name}: max error {err:.4g} vs max |ref| {scale:.4g}"


BWD_CASES = [
    # B, S, Hq, Hkv, d, w, lens, dt kind
    (2, 200, 4, 2, 64, 37, (200, 150), "lognormal"),
    (1, 130, 8, 1, 128, 200, None, "lognormal"),     # S <= w: every key kept
    (2, 333, 4, 1, 128, 50, (333, 100), "dyadic"),   # ties
    (3, 257, 2, 2, 64, 20, None, "wide"),
    (1, 300, 2, 2, 64, 1, None, "few"),              # w = 1
    (1, 190, 1, 1, 64, 64, None, "const"),           # G = 1, all dt equal
    (2, 97, 16, 2, 128, 33, (97, 1), "lognormal"),   # G = 8, a batch of length 1
    (2, 700, 4, 2, 128, 90, (700, 515), "wide"),     # several 128-key tiles, a length ending inside one
    (1, 300, 2, 2, 128, 40, None, "lognormal"),      # G = 1 at d = 128: row blocks of 64 rows
    (1, 2600, 4, 2, 64, 300, None, "lognormal"),     # query tiles past 1024 keys: several scan steps
    # late query tiles have more candidate keys than the query kernel's LDS
    # list holds and walk the causal range instead
    (1, 3300, 2, 1, 64, 3100, None, "lognormal"),
]


@pytest.mark.parametrize("B,S,Hq,Hkv,d,w,lens,kind", BWD_CASES)
def test_attn_bwd_elementwise(dma, oracle_mod, B, S, Hq, Hkv, d, w, lens, kind):
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", S + d)
    dO = si.make_qkv(B, S, Hq, Hkv, d, "bf16", S + d + 1)[0]
    dt = si.make_dt((B, Hkv, S), kind, S)
    seq = None if lens is None else np.array(lens, np.int32)
    q, k, v, dtd, sd = to_dev(Q), to_dev(K), to_dev(V), to_dev(dt), to_dev(seq)
    tau, tie = dma.select(dtd, w, sd)
    dQ, dK, dV, ddt = dma.attn_bwd(q, k, v, dtd, tau, tie, w, to_dev(dO), sd)
    torch.cuda.synchronize()
    rq, rk, rv, rd = oracle_mod.attn_bwd(Q, K, V, dt, w, dO, seq)
    _rel_check("dQ", to_host(dQ), rq, 2e-2)
    _rel_check("dK", to_host(dK), rk, 2e-2)
    _rel_check("dV", to_host(dV), rv, 2e-2)
    _rel_check("ddt", to_host(ddt), rd, 1e-3)
    if seq is not None:  # padded rows and keys are exact zeros
        for b, L in enumerate(seq):
            assert not to_host(dQ)[b, L:].any() and not to_host(dK)[b, L:].any()
            assert not to_host(dV)[b, L:].any() and not to_host(ddt)[b, :, L:].any()


def test_attn_bwd_deterministic_and_uniform_shift(dma, oracle_mod):
    B, S, Hq, Hkv, d, w = 2, 300, 8, 4, 64, 40
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", 21)
    dO = si.make_qkv(B, S, Hq, Hkv, d, "bf16", 22)[0]
    dt = si.make_dt((B, Hkv, S), "lognormal", 23)
    q, k, v, dtd, o = to_dev(Q), to_dev(K), to_dev(V), to_dev(dt), to_dev(dO)
    tau, tie = dma.select(dtd, w)
    a = dma.attn_bwd(q, k, v, dtd, tau, tie, w, o)
    b = dma.attn_bwd(q, k, v, dtd, tau, tie, w, o)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    # a uniform shift of dt changes nothing, so each (batch, kv head) row of
    # ddt sums to zero (up to float32 summation)
    ddt = to_host(a[3]).astype(np.float64)
    assert np.abs(ddt.sum(axis=2)).max() <= 1e-4 * np.abs(ddt).sum(axis=2).max()


def test_attn_bwd_full_size_c2(dma, oracle_mod):
    """The backward at the c2 workload's full size, every element."""
    wl = si.WORKLOADS["c2"]
    inp = si.make_inputs(wl)
    dO = si.make_qkv(wl.B, wl.S, wl.Hq, wl.Hkv, wl.d, "bf16", 31)[0]
    dt = oracle_mod.dt(inp["V"], inp["W"], inp["bias"], inp["A"]).astype(np.float32)
    dtd = to_dev(dt)
    tau, tie = dma.select(dtd, wl.w)
    dQ, dK, dV, ddt = dma.attn_bwd(to_dev(inp["Q"]), to_dev(inp["K"]), to_dev(inp["V"]), dtd, tau, tie, wl.w,
                                   to_dev(dO))
    torch.cuda.synchronize()
    rq, rk, rv, rd = oracle_mod.attn_bwd(inp["Q"], inp["K"], inp["V"], dt, wl.w, dO)
    _rel_check("dQ", to_host(dQ), rq, 2e-2)
    _rel_check("dK", to_host(dK), rk, 2e-2)
    _rel_check("dV", to_host(dV), rv, 2e-2)
    _rel_check("ddt", to_host(ddt), rd, 1e-3)


DT_CASES = [(2, 100, 4, 64, "bf16", True), (1, 67, 1, 64, "f32", False), (1, 130, 8, 128, "bf16", False),
            (3, 64, 2, 128, "f32", True),
            # more per-workgroup partial sums than the last level takes: one and two slice levels first
            (2, 1100, 2, 64, "bf16", True), (1, 17000, 1, 64, "f32", False)]


@pytest.mark.parametrize("B,S,Hkv,d,dtype,with_bias", DT_CASES)
def test_dt_bwd(dma, oracle_mod, B, S, Hkv, d, dtype, with_bias):
    inp = si.make_inputs(si.Workload("t", dtype, B, 2 * Hkv, Hkv, S, d, 8, seed=B * S + d))
    rng = np.random.default_rng(S)
    bias = si._store(rng.normal(0, 0.5, Hkv).astype(np.float32), dtype) if with_bias else None
    ddt = rng.standard_normal((B, Hkv, S)).astype(np.float32)
    X = si._store(rng.standard_normal((B, S, Hkv, d)).astype(np.float32), dtype)   # existing value gradient
    dV = to_dev(X)
    dW, db, dA = dma.dt_bwd(to_dev(inp["V"]), to_dev(inp["W"]), to_dev(inp["A"]), to_dev(ddt),
                            to_dev(bias), dV=dV)
    torch.cuda.synchronize()
    rv, rw, rb, ra = oracle_mod.dt_bwd(inp["V"], inp["W"], bias, inp["A"], ddt)
    _rel_check("dW", to_host(dW), rw, 1e-4)
    _rel_check("dbias", to_host(db), rb, 1e-4)
    _rel_check("dA", to_host(dA), ra, 1e-4)
    tot = host_f64(X) + rv
    half_ulp = 2.0 ** -8 * np.abs(tot) if dtype == "bf16" else 2e-7 * np.abs(tot)
    err = np.abs(to_host(dV).astype(np.float64) - tot)
    assert (err <= half_ulp + 1e-4 * np.abs(rv).max()).all(), err.max()


def test_prefill_bwd_chain(dma, oracle_mod):
    """attn_bwd -> dt_bwd (value gradient summed in place) against the
    oracle's chain, with the forward's dt taken from the oracle."""
    wl = si.Workload("chain", "bf16", 2, 8, 4, 260, 64, 48, pad_lo=130, pad_hi=260, seed=41)
    inp = si.make_inputs(wl)
    seq = inp["seqlens"]
    dO = si.make_qkv(wl.B, wl.S, wl.Hq, wl.Hkv, wl.d, "bf16", 42)[0]
    dt = oracle_mod.dt(inp["V"], inp["W"], inp["bias"], inp["A"]).astype(np.float32)
    dtd, sd = to_dev(dt), to_dev(seq)
    tau, tie = dma.select(dtd, wl.w, sd)
    g = dma.prefill_bwd(to_dev(inp["Q"]), to_dev(inp["K"]), to_dev(inp["V"]), to_dev(inp["W"]), to_dev(inp["A"]),
                        wl.w, to_dev(dO), bias=to_dev(inp["bias"]), seqlens=sd, fwd=(dtd, tau, tie))
    torch.cuda.synchronize()
    rq, rk, rv, rd = oracle_mod.attn_bwd(inp["Q"], inp["K"], inp["V"], dt, wl.w, dO, seq)
    rv2, rw, rb, ra = oracle_mod.dt_bwd(inp["V"], inp["W"], inp["bias"], inp["A"], rd)
    _rel_check("dQ", to_host(g["dQ"]), rq, 2e-2)
    _rel_check("dK", to_host(g["dK"]), rk, 2e-2)
    _rel_check("dV total", to_host(g["dV"]), rv + rv2, 2e-2)
    _rel_check("dW", to_host(g["dW"]), rw, 2e-3)
    _rel_check("dbias", to_host(g["dbias"]), rb, 2e-3)
    _rel_check("dA", to_host(g["dA"]), ra, 2e-3)

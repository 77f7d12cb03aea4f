"""GPU parity of the Q/K prologue: dma_qk_norm_rope and dma_prologue against the
CPU oracle (RMSNorm over head_dim, rotary embedding, dt) on the same seeded
inputs.

Bar.  The kernel works in float32 and rounds each output once; the oracle is
float64.  float32 outputs: |gpu - oracle| <= 2e-5 * (1 + |oracle|).  bf16
outputs: the final rounding moves a value by at most half a bf16 ulp, which
is at most 2^-8 of its magnitude, so |gpu - oracle| <= 2^-8 |oracle| + 2e-5
(the second term covers the float32 work before the rounding).  dt: rel 1e-5.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.gpu_util import host_f64, to_dev, to_host

pytestmark = pytest.mark.gpu

THETA = 10000.0
EPS = 1e-6


@pytest.fixture(scope="module")
def dma():
    import doge_dynamic_mask_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def _bound(dtype, ref):
    if dtype == "f32":
        return 2e-5 * (1.0 + np.abs(ref))
    return 2.0 ** -8 * np.abs(ref) + 2e-5


def _expect(oracle_mod, X, w, positions, eps=EPS, theta=THETA):
    """Oracle output of X [B, S, H, d] with one position per (b, s)."""
    B, S = X.shape[:2]
    pos = np.broadcast_to(np.arange(S, dtype=np.int32)[None, :], (B, S)) if positions is None else positions
    return oracle_mod.qk_norm_rope(X, w, eps, theta, pos[:, :, None])


def _check(dtype, got, ref, what):
    bad = np.abs(got - ref) > _bound(dtype, ref)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements off, first {i}: gpu {got[i]} oracle {ref[i]}")


CASES = [
    # dtype, B, S, Hq, Hkv, d, positions
    ("f32", 1, 37, 2, 1, 64, None),
    ("f32", 2, 19, 16, 8, 128, "offset"),
    ("f32", 3, 5, 3, 3, 64, "large"),
    ("bf16", 2, 45, 8, 4, 64, None),
    ("bf16", 1, 33, 16, 8, 128, "offset"),
    ("bf16", 2, 7, 5, 1, 128, "large"),        # rows past the last one in a step
    ("bf16", 1, 1, 1, 1, 64, "large"),          # one token
    ("bf16", 3, 11, 40, 8, 128, None),          # more rows than one batch of loads
    ("f32", 1, 9, 33, 11, 64, "offset"),
]


@pytest.mark.parametrize("dtype,B,S,Hq,Hkv,d,pk", CASES)
def test_qk_norm_rope_elementwise(dma, oracle_mod, dtype, B, S, Hq, Hkv, d, pk):
    seed = B * 1000 + S * 10 + Hq + d
    Q, K, _ = si.make_qkv(B, S, Hq, Hkv, d, dtype, seed)
    wq, wk = si.make_norm_weights(d, dtype, seed + 1)
    pos = None if pk is None else si.make_positions(B, S, pk, seed + 2)
    Qo, Ko = dma.qk_norm_rope(to_dev(Q), to_dev(K), to_dev(wq), to_dev(wk), EPS, THETA, to_dev(pos))
    torch.cuda.synchronize()
    _check(dtype, to_host(Qo), _expect(oracle_mod, Q, wq, pos), "Q")
    _check(dtype, to_host(Ko), _expect(oracle_mod, K, wk, pos), "K")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_qk_norm_rope_in_place_and_edges(dma, oracle_mod, dtype):
    B, S, Hq, Hkv, d = 2, 24, 8, 2, 128
    Q, K, _ = si.make_qkv(B, S, Hq, Hkv, d, dtype, 77)
    # zero rows normalise to zero; a row of one repeated value; tiny and large scales
    Qf, Kf = host_f64(Q).astype(np.float32), host_f64(K).astype(np.float32)
    Qf[0, 3, 2] = 0.0
    Kf[1, 5, 0] = 0.0
    Qf[1, 0, 1] = 2.5
    Qf[0, 7] *= 1e-12
    Kf[0, 9] *= 1e12
    Q, K = (Qf, Kf) if dtype == "f32" else (si.to_bf16_bits(Qf), si.to_bf16_bits(Kf))
    wq, wk = si.make_norm_weights(d, dtype, 78)
    pos = si.make_positions(B, S, "offset", 79)
    q, k = to_dev(Q), to_dev(K)
    Qo, Ko = dma.qk_norm_rope(q, k, to_dev(wq), to_dev(wk), EPS, THETA, to_dev(pos), Q_out=q, K_out=k)
    assert Qo.data_ptr() == q.data_ptr() and Ko.data_ptr() == k.data_ptr()
    torch.cuda.synchronize()
    rq, rk = _expect(oracle_mod, Q, wq, pos), _expect(oracle_mod, K, wk, pos)
    _check(dtype, to_host(q), rq, "Q in place")
    _check(dtype, to_host(k), rk, "K in place")
    assert not to_host(q)[0, 3, 2].any() and not to_host(k)[1, 5, 0].any()


def test_qk_norm_rope_eps_theta_and_position_zero(dma, oracle_mod):
    # eps = 0.3 and theta = 500: other parameters than the defaults; position
    # 0 everywhere leaves RMSNorm alone
    B, S, Hq, Hkv, d = 1, 16, 4, 2, 64
    Q, K, _ = si.make_qkv(B, S, Hq, Hkv, d, "f32", 80)
    wq, wk = si.make_norm_weights(d, "f32", 81)
    pos = si.make_positions(B, S, "large", 82)
    Qo, Ko = dma.qk_norm_rope(to_dev(Q), to_dev(K), to_dev(wq), to_dev(wk), 0.3, 500.0, to_dev(pos))
    torch.cuda.synchronize()
    _check("f32", to_host(Qo), _expect(oracle_mod, Q, wq, pos, 0.3, 500.0), "Q")
    _check("f32", to_host(Ko), _expect(oracle_mod, K, wk, pos, 0.3, 500.0), "K")
    zero = np.zeros((B, S), np.int32)
    Qo, _ = dma.qk_norm_rope(to_dev(Q), to_dev(K), to_dev(wq), to_dev(wk), EPS, THETA, to_dev(zero))
    torch.cuda.synchronize()
    x = Q.astype(np.float64)
    norm = x / np.sqrt((x ** 2).mean(-1, keepdims=True) + EPS) * wq
    _check("f32", to_host(Qo), norm, "Q at position 0")


def _dt_check(oracle_mod, inp, got):
    ref = oracle_mod.dt(inp["V"], inp["W"], inp["bias"], inp["A"])
    rel = np.abs(got - ref) / np.abs(ref)
    assert rel.max() <= 1e-5, rel.max()


@pytest.mark.parametrize("name,tokens", [("c2", None), ("long", 512), ("padded", 256)])
def test_prologue_full_size(dma, oracle_mod, name, tokens):
    """dma_prologue at a workload's full size, launched as the benchmark does:
    Q/K compared with the oracle on every token (c2) or on sampled tokens,
    dt on every position."""
    inp = si.make_inputs(si.WORKLOADS[name])
    wl = si.WORKLOADS[name]
    wq, wk = si.make_norm_weights(wl.d, wl.dtype, wl.seed + 7)
    Qd, Kd, Vd = to_dev(inp["Q"]), to_dev(inp["K"]), to_dev(inp["V"])
    Qo, Ko, dt = dma.prologue(Qd, Kd, Vd, to_dev(wq), to_dev(wk), to_dev(inp["W"]), to_dev(inp["A"]),
                              to_dev(inp["bias"]))
    torch.cuda.synchronize()
    dt_plain = dma.dt(Vd, to_dev(inp["W"]), to_dev(inp["A"]), to_dev(inp["bias"]))
    torch.cuda.synchronize()
    assert torch.equal(dt, dt_plain)
    _dt_check(oracle_mod, inp, to_host(dt))
    B, S = wl.B, wl.S
    if tokens is None:
        bs = np.array([(b, s) for b in range(B) for s in range(S)])
    else:
        rng = np.random.default_rng(wl.seed + 8)
        bs = np.stack([rng.integers(B, size=tokens), rng.integers(S, size=tokens)], 1)
        bs = np.concatenate([bs, [[0, 0], [B - 1, S - 1]]])
    gq, gk = to_host(Qo), to_host(Ko)
    for X, w, got, what in ((inp["Q"], wq, gq, "Q"), (inp["K"], wk, gk, "K")):
        rows = X[bs[:, 0], bs[:, 1]]                              # [n, H, d]
        ref = oracle_mod.qk_norm_rope(rows, w, EPS, THETA, bs[:, 1][:, None])
        _check(wl.dtype, got[bs[:, 0], bs[:, 1]], ref, what)


def test_prologue_decode_token(dma, oracle_mod):
    """One decode token per batch (S = 1) at position L_b, as the incremental
    path feeds it: positions [B, 1]."""
    B, Hq, Hkv, d = 8, 8, 2, 128
    Q, K, V = si.make_qkv(B, 1, Hq, Hkv, d, "bf16", 90)
    wq, wk = si.make_norm_weights(d, "bf16", 91)
    lens = si.make_lengths(B, 1, 16384, 92).reshape(B, 1)
    inp = si.make_inputs(si.WORKLOADS["decode"], B=B, S=1)
    Qo, Ko, dt = dma.prologue(to_dev(Q), to_dev(K), to_dev(V), to_dev(wq), to_dev(wk), to_dev(inp["W"]),
                              to_dev(inp["A"]), None, positions=to_dev(lens))
    torch.cuda.synchronize()
    _check("bf16", to_host(Qo), _expect(oracle_mod, Q, wq, lens), "q")
    _check("bf16", to_host(Ko), _expect(oracle_mod, K, wk, lens), "k")
    _dt_check(oracle_mod, {"V": V, "W": inp["W"], "A": inp["A"], "bias": None}, to_host(dt))
    # a call this small takes the one-wave-per-(token, head) dt path in both
    # entry points: the same bits
    dt_plain = dma.dt(to_dev(V), to_dev(inp["W"]), to_dev(inp["A"]), None)
    torch.cuda.synchronize()
    assert torch.equal(dt, dt_plain)


@pytest.mark.parametrize("B,S,Hkv,d", [(2, 50, 4, 64), (1, 256, 16, 128), (1, 257, 3, 128)])
def test_prologue_dt_matches_dma_dt_small(dma, oracle_mod, B, S, Hkv, d):
    """Calls around the small-call threshold (256 tokens): dma_prologue's dt
    is bit-identical to dma_dt's and within the oracle's tolerance."""
    Hq = 2 * Hkv
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", 93 + S)
    wq, wk = si.make_norm_weights(d, "bf16", 94)
    rng = np.random.default_rng(95 + S)
    W = si.to_bf16_bits(rng.normal(0, 0.02, (Hkv, Hkv * d)).astype(np.float32))
    A = rng.uniform(-2, 2, Hkv).astype(np.float32)
    bias = si.to_bf16_bits(rng.normal(0, 0.5, Hkv).astype(np.float32))
    _, _, dt = dma.prologue(to_dev(Q), to_dev(K), to_dev(V), to_dev(wq), to_dev(wk), to_dev(W), to_dev(A),
                            to_dev(bias))
    dt_plain = dma.dt(to_dev(V), to_dev(W), to_dev(A), to_dev(bias))
    torch.cuda.synchronize()
    assert torch.equal(dt, dt_plain)
    _dt_check(oracle_mod, {"V": V, "W": W, "A": A, "bias": bias}, to_host(dt))

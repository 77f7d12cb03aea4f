"""Pins of the oracle's gradients (CPU): oracle.attn_bwd and oracle.dt_bwd.

Each test checks the gradients against something other than their own
formulas: central finite differences of the pinned forward oracle (on inputs
from a dyadic grid, so that every perturbed input is exact in float32, and
with dt values spaced far wider than the step, so that no kept set changes),
torch autograd through a dense masked-softmax formulation written in torch,
and invariants of the method (a uniform shift of dt changes nothing, so the
dt gradients of a (batch, kv head) row sum to zero; a row that keeps one key
passes dO straight to that key's value).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si


def _grid(rng, shape, scale=16):
    """N(0, 1) draws rounded to multiples of 1/scale (exact in float32)."""
    return (np.round(rng.standard_normal(shape) * scale) / scale).astype(np.float32)


def _spaced_dt(rng, B, Hkv, S):
    """Distinct dt values 0.5 + k/8 in random order per row: ties never occur and
    a step of 2^-10 never reorders keys."""
    out = np.empty((B, Hkv, S), np.float32)
    for b in range(B):
        for g in range(Hkv):
            out[b, g] = 0.5 + rng.permutation(S) / 8.0
    return out


def _loss(Q, K, V, dt, w, dO, seqlens):
    return float((oracle.attn(Q, K, V, dt, w, seqlens) * dO.astype(np.float64)).sum())


@pytest.mark.parametrize("B,S,Hq,Hkv,d,w,padded", [(1, 10, 2, 1, 8, 4, False), (2, 9, 4, 2, 8, 3, True)])
def test_attn_bwd_finite_differences(B, S, Hq, Hkv, d, w, padded):
    rng = np.random.default_rng(S * 10 + w)
    Q, K, V = _grid(rng, (B, S, Hq, d)), _grid(rng, (B, S, Hkv, d)), _grid(rng, (B, S, Hkv, d))
    dt = _spaced_dt(rng, B, Hkv, S)
    dO = _grid(rng, (B, S, Hq, d))
    seq = np.array([S, S - 3][:B], np.int32) if padded else None
    dQ, dK, dV, ddt = oracle.attn_bwd(Q, K, V, dt, w, dO, seq)
    h = 2.0 ** -10
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV), ("dt", dt, ddt)):
        fd = np.empty(X.shape)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args = {"Q": Q, "K": K, "V": V, "dt": dt}
            args[name] = Xp
            fp = _loss(args["Q"], args["K"], args["V"], args["dt"], w, dO, seq)
            args[name] = Xm
            fm = _loss(args["Q"], args["K"], args["V"], args["dt"], w, dO, seq)
            fd[idx] = (fp - fm) / (2 * h)
        assert np.allclose(G, fd, rtol=1e-5, atol=1e-6), (name, np.abs(G - fd).max())


def _dense_torch(Q, K, V, dt, w, dO, seqlens):
    """Autograd of the masked softmax written densely in torch (fp64): the kept
    mask from oracle.kept_row, -inf elsewhere."""
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    mask = np.zeros((B, Hkv, S, S), bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(S):
                if seqlens is None or i < seqlens[b]:
                    mask[b, g, i, oracle.kept_row(dt, w, b, g, i, seqlens)] = True
    q = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    t = torch.tensor(dt, dtype=torch.float64, requires_grad=True)
    kk = k.repeat_interleave(G, dim=2)            # [B, S, Hq, d]
    vv = v.repeat_interleave(G, dim=2)
    tt = t.repeat_interleave(G, dim=1)            # [B, Hq, S]
    mm = torch.tensor(mask).repeat_interleave(G, dim=1)
    s = torch.einsum("bihd,bjhd->bhij", q, kk) / np.sqrt(d) + tt[:, :, None, :]
    s = s.masked_fill(~mm, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)              # padded rows keep nothing
    o = torch.einsum("bhij,bjhd->bihd", p, vv)
    (o * torch.tensor(dO, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), t.grad.numpy()


@pytest.mark.parametrize("kind,padded", [("lognormal", False), ("few", True), ("const", False)])
def test_attn_bwd_matches_dense_autograd(kind, padded):
    B, S, Hq, Hkv, d, w = 2, 40, 4, 2, 16, 9
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "f32", 3)
    dO = si.make_qkv(B, S, Hq, Hkv, d, "f32", 4)[0]
    dt = si.make_dt((B, Hkv, S), kind, 5)
    seq = si.make_lengths(B, 20, S, 6) if padded else None
    got = oracle.attn_bwd(Q, K, V, dt, w, dO, seq)
    ref = _dense_torch(Q, K, V, dt, w, dO, seq)
    for name, a, r in zip(("dQ", "dK", "dV", "ddt"), got, ref):
        assert np.allclose(a, r, rtol=1e-10, atol=1e-12), (name, np.abs(a - r).max())


def test_attn_bwd_invariants():
    B, S, Hq, Hkv, d, w = 2, 64, 4, 2, 16, 11
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", 7)
    dO = si.make_qkv(B, S, Hq, Hkv, d, "bf16", 8)[0]
    dt = si.make_dt((B, Hkv, S), "dyadic", 9)
    seq = np.array([64, 50], np.int32)
    dQ, dK, dV, ddt = oracle.attn_bwd(Q, K, V, dt, w, dO, seq)
    # a uniform shift of a row's dt leaves every output unchanged
    assert np.abs(ddt.sum(axis=2)).max() < 1e-10
    # padded keys and rows get nothing
    assert not ddt[1, :, 50:].any() and not dK[1, 50:].any() and not dV[1, 50:].any() and not dQ[1, 50:].any()
    # w = 1: each row keeps one key, its softmax is constant, so dQ = ddt = 0 and
    # that key's value gradient is the sum of dO over the rows that keep it
    dQ1, dK1, dV1, ddt1 = oracle.attn_bwd(Q, K, V, dt, 1, dO, seq)
    assert not dQ1.any() and not dK1.any() and not ddt1.any()
    G = Hq // Hkv
    dOf = si.bf16_bits_to_f32(dO).astype(np.float64)
    expect = np.zeros_like(dV1)
    for b in range(B):
        for g in range(Hkv):
            for i in range(seq[b]):
                j = oracle.kept_row(dt, 1, b, g, i, seq)[0]
                expect[b, j, g] += dOf[b, i, g * G:(g + 1) * G].sum(axis=0)
    assert np.allclose(dV1, expect, rtol=0, atol=1e-12)


def _dt_loss(V, W, bias, A, ddt):
    return float((oracle.dt(V, W, bias, A) * ddt).sum())


def test_dt_bwd_finite_differences():
    rng = np.random.default_rng(11)
    B, S, Hkv, d = 2, 3, 2, 4
    V = _grid(rng, (B, S, Hkv, d), 8)
    W = _grid(rng, (Hkv, Hkv * d), 64)
    bias = _grid(rng, (Hkv,), 8)
    A = np.array([0.75, -1.25], np.float32)
    ddt = rng.standard_normal((B, Hkv, S))
    dV, dW, dbias, dA = oracle.dt_bwd(V, W, bias, A, ddt)
    h = 2.0 ** -12
    for name, X, G in (("V", V, dV), ("W", W, dW), ("bias", bias, dbias), ("A", A, dA)):
        fd = np.empty(X.shape)
        for idx in np.ndindex(X.shape):
            args = {"V": V, "W": W, "bias": bias, "A": A}
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args[name] = Xp
            fp = _dt_loss(args["V"], args["W"], args["bias"], args["A"], ddt)
            args[name] = Xm
            fm = _dt_loss(args["V"], args["W"], args["bias"], args["A"], ddt)
            fd[idx] = (fp - fm) / (2 * h)
        assert np.allclose(G, fd, rtol=1e-6, atol=1e-8), (name, np.abs(G - fd).max())


@pytest.mark.parametrize("with_bias", [True, False])
def test_dt_bwd_matches_autograd(with_bias):
    B, S, Hkv, d = 2, 17, 4, 16
    inp = si.make_inputs(si.Workload("t", "bf16", B, 2 * Hkv, Hkv, S, d, 8, seed=12))
    rng = np.random.default_rng(13)
    bias = si.to_bf16_bits(rng.normal(0, 0.5, Hkv).astype(np.float32)) if with_bias else None
    ddt = rng.standard_normal((B, Hkv, S))
    got = oracle.dt_bwd(inp["V"], inp["W"], bias, inp["A"], ddt)
    v = torch.tensor(si.bf16_bits_to_f32(inp["V"]), dtype=torch.float64, requires_grad=True)
    W = torch.tensor(si.bf16_bits_to_f32(inp["W"]), dtype=torch.float64, requires_grad=True)
    A = torch.tensor(inp["A"], dtype=torch.float64, requires_grad=True)
    bb = torch.tensor(si.bf16_bits_to_f32(bias) if with_bias else np.zeros(Hkv, np.float32),
                      dtype=torch.float64, requires_grad=True)
    x = v.reshape(B, S, Hkv * d) @ W.T + bb           # [B, S, Hkv]
    dtv = torch.exp(A * torch.nn.functional.softplus(x))
    (dtv.permute(0, 2, 1) * torch.tensor(ddt)).sum().backward()
    ref = (v.grad.numpy(), W.grad.numpy(), bb.grad.numpy(), A.grad.numpy())
    for name, a, r in zip(("dV", "dW", "dbias", "dA"), got, ref):
        assert np.allclose(a, r, rtol=1e-10, atol=1e-12), (name, np.abs(a - r).max())

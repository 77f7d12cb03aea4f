"""Pins of the oracle's CDMoE routed experts (CPU).

(The routing from given float32 logits ranks a pair on the float32 sum of its
two logits, the precision the GPU kernel decides in; the brute force below
does the same.)

The two-stage product-key routing (top k per domain, then the top k of the
k*k pairs) is checked against a brute force that scores every one of the
nk*nk experts directly (score = x logit + y logit) and sorts them all, equal
scores in the order of the two domains' own rankings (the x key's rank, then
the y key's); the weights against the softmax closed form; the logits
against a library matmul; the expert output against a dense formulation
that weights every expert (zero for the ones not kept).
"""
import numpy as np
import pytest

import synth_inputs as si


def _domain_rank(v):
    """rank of each key in its domain: larger first, lower index first among equal"""
    order = np.lexsort((np.arange(v.size), -v))
    r = np.empty(v.size, np.int64)
    r[order] = np.arange(v.size)
    return r


def _brute_route(logits, k):
    T, n2 = logits.shape
    nk = n2 // 2
    lx, ly = logits[:, :nk].astype(np.float32), logits[:, nk:].astype(np.float32)
    idx = np.empty((T, k), np.int64)
    sc = np.empty((T, k))
    for t in range(T):
        # expert a*nk + b scores the float32 sum of its two logits
        s = (lx[t][:, None] + ly[t][None, :]).reshape(-1).astype(np.float64)
        tie = (_domain_rank(lx[t])[:, None] * nk + _domain_rank(ly[t])[None, :]).reshape(-1)
        order = np.lexsort((tie, -s))                        # score desc, then the domain ranks
        idx[t] = order[:k]
        sc[t] = s[order[:k]]
    return idx, sc


@pytest.mark.parametrize("nk,k,kind", [(8, 3, "normal"), (16, 16, "normal"), (12, 5, "few"), (11, 1, "few"),
                                       (128, 64, "normal")])
def test_route_equals_global_topk_over_all_experts(oracle_mod, nk, k, kind):
    rng = np.random.default_rng(nk * 100 + k)
    T = 7
    if kind == "few":     # many exact ties, resolved by the lower expert index
        logits = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(T, 2 * nk))
    else:
        logits = rng.standard_normal((T, 2 * nk)).astype(np.float32)
    idx, wts = oracle_mod.cdmoe_route(logits, k)
    bidx, bsc = _brute_route(logits, k)
    assert np.array_equal(idx, bidx)
    ref_w = np.exp(bsc - bsc.max(axis=1, keepdims=True))
    ref_w /= ref_w.sum(axis=1, keepdims=True)
    assert np.allclose(wts, ref_w, rtol=1e-14, atol=0)
    assert np.allclose(wts.sum(axis=1), 1.0, rtol=1e-14)


def _silu(z):
    return z / (1.0 + np.exp(-z))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cdmoe_output_against_dense_formulation(oracle_mod, dtype):
    T, H, nk, k = 6, 48, 9, 4
    h, router, down, up = si.make_cdmoe(T, H, nk, dtype, seed=3)
    idx, wts, out = oracle_mod.cdmoe(h, router, down, up, k)
    f = (lambda x: si.bf16_bits_to_f32(x).astype(np.float64)) if dtype == "bf16" else (lambda x: x.astype(np.float64))
    hf, rf, df, uf = f(h), f(router), f(down), f(up)
    logits = hf @ rf.T                                    # library matmul
    # the kept experts are the global top k of all nk*nk scores (fp64 logits)
    for t in range(T):
        s = (logits[t, :nk][:, None] + logits[t, nk:][None, :]).reshape(-1)
        tie = (_domain_rank(logits[t, :nk])[:, None] * nk + _domain_rank(logits[t, nk:])[None, :]).reshape(-1)
        order = np.lexsort((tie, -s))[:k]
        assert idx[t].tolist() == order.tolist()
        wdense = np.zeros(nk * nk)
        e = np.exp(s[order] - s[order].max())
        wdense[order] = e / e.sum()
        ref = (wdense * _silu(df @ hf[t])) @ uf            # every expert, zero weight unless kept
        assert np.allclose(out[t], ref, rtol=1e-10, atol=1e-12)
        assert np.allclose(wts[t], wdense[order], rtol=1e-12)


def test_single_expert_gets_weight_one(oracle_mod):
    T, H, nk = 3, 16, 5
    h, router, down, up = si.make_cdmoe(T, H, nk, "f32", seed=4)
    idx, wts, out = oracle_mod.cdmoe(h, router, down, up, 1)
    assert np.array_equal(wts, np.ones((T, 1)))
    for t in range(T):
        e = idx[t, 0]
        z = float(down[e].astype(np.float64) @ h[t].astype(np.float64))
        assert np.allclose(out[t], _silu(z) * up[e].astype(np.float64), rtol=1e-12, atol=1e-14)


def test_logits_and_experts_alone(oracle_mod):
    """The two halves exported on their own: logits against a library matmul,
    experts against the dense all-expert formulation for arbitrary (also
    repeated) expert lists and weights, and both against the whole oracle."""
    T, H, nk, k = 5, 32, 6, 3
    h, router, down, up = si.make_cdmoe(T, H, nk, "bf16", seed=8)
    f = lambda x: si.bf16_bits_to_f32(x).astype(np.float64)
    lg = oracle_mod.cdmoe_logits(h, router)
    assert np.allclose(lg, f(h) @ f(router).T, rtol=1e-12, atol=1e-15)
    rng = np.random.default_rng(9)
    idx = rng.integers(0, nk * nk, size=(T, k)).astype(np.int32)
    idx[0, 1] = idx[0, 0]                                   # a repeated expert adds twice
    w = rng.random((T, k))
    got = oracle_mod.cdmoe_experts(h, down, up, idx, w)
    for t in range(T):
        wd = np.zeros(nk * nk)
        np.add.at(wd, idx[t], w[t])
        assert np.allclose(got[t], (wd * _silu(f(down) @ f(h)[t])) @ f(up), rtol=1e-10, atol=1e-14)
    i2, w2, o2 = oracle_mod.cdmoe(h, router, down, up, k)
    assert np.allclose(oracle_mod.cdmoe_experts(h, down, up, i2, w2), o2, rtol=1e-12, atol=1e-15)

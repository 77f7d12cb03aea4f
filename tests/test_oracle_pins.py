"""Pins of the CPU oracle against closed forms, library routines and invariants.

Nothing here re-types the oracle's formulas: each check is an identity or a
special case that the Doge guide's DMA definition (gitcode page, section on
Dynamic Mask Attention, forward steps 3-4) reduces to, or a library routine
(numpy matmul, torch SDPA on the CPU).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------- dt
def _dt_inputs(dtype, B=2, S=9, Hkv=3, d=8, seed=0):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((B, S, Hkv, d)).astype(np.float32)
    W = rng.normal(0, 0.3, size=(Hkv, Hkv * d)).astype(np.float32)
    b = rng.normal(0, 0.5, size=Hkv).astype(np.float32)
    A = rng.uniform(-2, 2, size=Hkv).astype(np.float32)
    if dtype == "bf16":
        V, W, b = si.to_bf16_bits(V), si.to_bf16_bits(W), si.to_bf16_bits(b)
    return V, W, b, A


def _f(x):
    return si.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dt_zero_projection_is_two_to_the_A(oracle_mod, dtype):
    # softplus(0) = ln 2, so dt = exp(A ln 2) = 2^A whatever V holds.
    V, W, _, A = _dt_inputs(dtype)
    W = np.zeros_like(W)
    out = oracle_mod.dt(V, W, None, A)
    want = np.power(2.0, A.astype(np.float64))[None, :, None]
    np.testing.assert_allclose(out, np.broadcast_to(want, out.shape), rtol=1e-14, atol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dt_A_zero_is_one(oracle_mod, dtype):
    V, W, b, A = _dt_inputs(dtype)
    out = oracle_mod.dt(V, W, b, np.zeros_like(A))
    assert np.all(out == 1.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dt_inverts_to_library_matmul(oracle_mod, dtype):
    # Undo exp and softplus in closed form and compare the recovered
    # pre-activation with numpy's matmul of the concatenated-head value states
    # (input width Hkv*d, one output per kv head).  A transposed W, a wrong
    # head-major index or a dropped bias fails here.
    V, W, b, A = _dt_inputs(dtype, seed=3)
    out = oracle_mod.dt(V, W, b, A)
    B, S, Hkv, d = V.shape
    x_lib = _f(V).astype(np.float64).reshape(B, S, Hkv * d) @ _f(W).astype(np.float64).T
    x_lib = x_lib + _f(b).astype(np.float64)
    sp = np.log(out) / A.astype(np.float64)[None, :, None]      # softplus(x)
    x_rec = np.log(np.expm1(sp))                               # softplus^-1
    np.testing.assert_allclose(x_rec.transpose(0, 2, 1), x_lib, rtol=1e-9, atol=1e-9)


def test_dt_one_hot_reads_one_weight_and_softplus_symmetry(oracle_mod):
    # V one-hot at flat column c with value +v or -v: x = +-W[h, c] * v, and
    # softplus(x) - softplus(-x) = x gives log(dt+) - log(dt-) = A * W[h,c] * v.
    Hkv, d = 3, 8
    rng = np.random.default_rng(7)
    W = rng.normal(0, 0.7, size=(Hkv, Hkv * d)).astype(np.float32)
    A = np.array([1.5, -0.75, 0.3], dtype=np.float32)
    for c in (0, 5, d, 2 * d + 3):
        V = np.zeros((1, 2, Hkv, d), np.float32)
        V.reshape(1, 2, Hkv * d)[0, 0, c] = 1.25
        V.reshape(1, 2, Hkv * d)[0, 1, c] = -1.25
        out = oracle_mod.dt(V, W, None, A)
        lhs = np.log(out[0, :, 0]) - np.log(out[0, :, 1])
        rhs = A.astype(np.float64) * W[:, c].astype(np.float64) * 1.25
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-15)


def test_dt_softplus_tails(oracle_mod):
    # softplus(x) -> x for large x and -> e^x for very negative x.
    Hkv, d = 1, 4
    W = np.zeros((1, 4), np.float32)
    W[0, 0] = 1.0
    A = np.array([0.5], np.float32)
    V = np.zeros((1, 2, 1, 4), np.float32)
    V[0, 0, 0, 0] = 40.0
    V[0, 1, 0, 0] = -40.0
    out = oracle_mod.dt(V, W, None, A)
    assert out[0, 0, 0] == pytest.approx(math.exp(0.5 * 40.0), rel=1e-15)
    assert out[0, 0, 1] == pytest.approx(1.0 + 0.5 * math.exp(-40.0), rel=1e-15)


# ----------------------------------------------------------------- select
def test_select_golden_worked_example(oracle_mod):
    with open(os.path.join(GOLDEN, "select_worked_example.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        dt = np.array(case["dt"], np.float32)[None, None, :]
        seq = None if case.get("length") is None else np.array([case["length"]], np.int32)
        tau, tie = oracle_mod.select(dt, case["w"], seq)
        for i, (t, k) in enumerate(zip(case["tau"], case["tie"])):
            want = {"-inf": -np.inf, "+inf": np.inf}.get(t, t)
            assert tau[0, 0, i] == np.float32(want), (case["name"], i)
            assert tie[0, 0, i] == k, (case["name"], i)
        for i, ks in enumerate(case["kept"]):
            got = oracle_mod.kept_row(dt, case["w"], 0, 0, i, seq)
            assert got.tolist() == ks, (case["name"], i)


def _kept_matrix(oracle_mod, dt, w, seq):
    B, Hkv, S = dt.shape
    K = np.zeros((B, Hkv, S, S), bool)
    for b in range(B):
        for g in range(Hkv):
            for i in range(S):
                K[b, g, i, oracle_mod.kept_row(dt, w, b, g, i, seq)] = True
    return K


@pytest.mark.parametrize("kind", ["lognormal", "dyadic", "few", "const", "wide"])
def test_select_invariants(oracle_mod, kind):
    B, Hkv, S, w = 2, 2, 300, 37
    dt = si.make_dt((B, Hkv, S), kind, seed=11)
    seq = np.array([300, 171], np.int32)
    tau, tie = oracle_mod.select(dt, w, seq)
    K = _kept_matrix(oracle_mod, dt, w, seq)
    for b in range(B):
        L = seq[b]
        for g in range(Hkv):
            for i in range(S):
                if i >= L:
                    assert tau[b, g, i] == np.inf and tie[b, g, i] == -1
                    assert not K[b, g, i].any()
                    continue
                assert K[b, g, i].sum() == min(i + 1, w)
                assert not K[b, g, i, i + 1:].any()
                # the threshold test reproduces the kept set
                j = np.arange(i + 1)
                d = dt[b, g, : i + 1]
                test = (d > tau[b, g, i]) | ((d == tau[b, g, i]) & (j <= tie[b, g, i]))
                assert (test == K[b, g, i, : i + 1]).all()
                if i > 0:
                    # nesting: kept_i is inside kept_{i-1} plus {i}
                    prev = K[b, g, i - 1].copy()
                    prev[i] = True
                    assert not (K[b, g, i] & ~prev).any()
                    # (tau, -t) is nondecreasing once rows hold more than w keys
                    if i >= w + 1:
                        a = (tau[b, g, i - 1], -tie[b, g, i - 1])
                        c = (tau[b, g, i], -tie[b, g, i])
                        assert a <= c


def test_select_constant_dt_keeps_first_w(oracle_mod):
    # A = 0 makes every dt equal; the lower-index rule keeps keys 0..w-1.
    S, w = 200, 50
    dt = np.ones((1, 1, S), np.float32)
    tau, tie = oracle_mod.select(dt, w)
    for i in range(S):
        if i + 1 <= w:
            assert tau[0, 0, i] == -np.inf
        else:
            assert tau[0, 0, i] == 1.0 and tie[0, 0, i] == w - 1
            assert oracle_mod.kept_row(dt, w, 0, 0, i).tolist() == list(range(w))


def test_select_w1_is_running_argmax(oracle_mod):
    dt = si.make_dt((1, 1, 500), "few", seed=5)
    tau, tie = oracle_mod.select(dt, 1)
    x = dt[0, 0].astype(np.float64)
    for i in range(1, 500):
        j = int(np.argmax(x[: i + 1]))  # numpy argmax returns the first maximum
        assert tie[0, 0, i] == j and tau[0, 0, i] == dt[0, 0, j]


def test_select_scale_by_two_keeps_indices(oracle_mod):
    dt = si.make_dt((2, 3, 400), "lognormal", seed=9)
    _, t1 = oracle_mod.select(dt, 60)
    _, t2 = oracle_mod.select(dt * np.float32(2.0), 60)
    assert (t1 == t2).all()


def test_select_row_list_matches_full(oracle_mod):
    dt = si.make_dt((2, 2, 257), "dyadic", seed=4)
    seq = np.array([257, 100], np.int32)
    tau, tie = oracle_mod.select(dt, 31, seq)
    rows = np.array([(b, g, i) for b in range(2) for g in range(2) for i in (0, 30, 31, 99, 100, 256)])
    t2, i2 = oracle_mod.select(dt, 31, seq, rows=rows)
    for k, (b, g, i) in enumerate(rows):
        assert t2[k] == tau[b, g, i] and i2[k] == tie[b, g, i]


# -------------------------------------------------------------- attention
def _floats(x):
    return _f(x).astype(np.float64)


def _sdpa(Qf, Kf, Vf, mask_bgij, G):
    # torch SDPA (CPU, fp64) with a float additive mask, per kv-head group.
    q = torch.from_numpy(Qf).permute(0, 2, 1, 3)
    k = torch.from_numpy(np.repeat(Kf, G, axis=2)).permute(0, 2, 1, 3)
    v = torch.from_numpy(np.repeat(Vf, G, axis=2)).permute(0, 2, 1, 3)
    m = torch.from_numpy(np.repeat(mask_bgij, G, axis=1))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attn_dense_case_matches_library_sdpa(oracle_mod, dtype):
    # When no row has more than w valid keys, DMA is dense causal attention
    # with dt as an additive bias.
    B, S, Hq, Hkv, d = 2, 40, 4, 2, 16
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, dtype, seed=1)
    dt = si.make_dt((B, Hkv, S), "lognormal", seed=2)
    out = oracle_mod.attn(Q, K, V, dt, w=S)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = np.where(j <= i, dt[:, :, None, :].astype(np.float64), -np.inf)
    ref = _sdpa(_floats(Q), _floats(K), _floats(V), m, Hq // Hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_attn_constant_dt_is_causal_over_first_w(oracle_mod):
    # A = 0: dt == 1 everywhere, the kept set is keys 0..min(i, w-1) and the
    # uniform bias cancels in the softmax.
    B, S, Hq, Hkv, d, w = 1, 64, 2, 1, 8, 20
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "f32", seed=3)
    dt = np.ones((B, Hkv, S), np.float32)
    out = oracle_mod.attn(Q, K, V, dt, w)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = np.where(j <= np.minimum(i, w - 1), 0.0, -np.inf)[None, None]
    ref = _sdpa(_floats(Q), _floats(K), _floats(V), m, Hq // Hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_attn_w1_copies_argmax_value(oracle_mod):
    B, S, Hq, Hkv, d = 1, 50, 2, 1, 8
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", seed=4)
    dt = si.make_dt((B, Hkv, S), "few", seed=6)
    out = oracle_mod.attn(Q, K, V, dt, w=1)
    Vf = _floats(V)
    for i in range(S):
        j = int(np.argmax(dt[0, 0, : i + 1]))
        for hq in range(Hq):
            assert (out[0, i, hq] == Vf[0, j, 0]).all()


def test_attn_uniform_bias_invariance(oracle_mod):
    B, S, Hq, Hkv, d, w = 1, 120, 2, 1, 16, 30
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "f32", seed=8)
    dt = si.make_dt((B, Hkv, S), "dyadic", seed=10)     # exact under the shift
    o1 = oracle_mod.attn(Q, K, V, dt, w)
    o2 = oracle_mod.attn(Q, K, V, dt + np.float32(37 * 2.0 ** -10), w)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


def test_attn_gqa_equals_mha_with_repeated_heads(oracle_mod):
    B, S, Hq, Hkv, d, w = 1, 90, 6, 2, 8, 25
    G = Hq // Hkv
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", seed=12)
    dt = si.make_dt((B, Hkv, S), "lognormal", seed=13)
    o1 = oracle_mod.attn(Q, K, V, dt, w)
    o2 = oracle_mod.attn(Q, np.repeat(K, G, axis=2), np.repeat(V, G, axis=2),
                         np.repeat(dt, G, axis=1), w)
    assert (o1 == o2).all()


def test_attn_padding_equals_truncated_run(oracle_mod):
    B, S, Hq, Hkv, d, w = 2, 80, 4, 2, 8, 16
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "f32", seed=14)
    dt = si.make_dt((B, Hkv, S), "lognormal", seed=15)
    seq = np.array([80, 53], np.int32)
    Kn, Vn = K.copy(), V.copy()
    Kn[1, 53:] = np.nan
    Vn[1, 53:] = np.nan
    dtn = dt.copy()
    dtn[1, :, 53:] = np.nan
    out = oracle_mod.attn(Q, Kn, Vn, dtn, w, seqlens=seq)
    assert np.isfinite(out).all()
    assert (out[1, 53:] == 0).all()
    ref = oracle_mod.attn(Q[1:, :53], K[1:, :53], V[1:, :53], dt[1:, :, :53], w)
    np.testing.assert_array_equal(out[1:, :53], ref)


def test_decode_equals_last_prefill_row(oracle_mod):
    B, S, Hq, Hkv, d, w = 3, 70, 4, 2, 8, 19
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "bf16", seed=16)
    dt = si.make_dt((B, Hkv, S), "dyadic", seed=17)
    lens = np.array([70, 19, 44], np.int32)
    full = oracle_mod.attn(Q, K, V, dt, w, seqlens=lens)
    q = np.stack([Q[b, lens[b] - 1] for b in range(B)])
    out, kept = oracle_mod.decode(q, K, V, dt, lens, w)
    for b in range(B):
        np.testing.assert_array_equal(out[b], full[b, lens[b] - 1])
        for g in range(Hkv):
            ks = oracle_mod.kept_row(dt, w, b, g, lens[b] - 1, lens)
            got = kept[b, g]
            assert got[: len(ks)].tolist() == ks.tolist()
            assert (got[len(ks):] == -1).all()

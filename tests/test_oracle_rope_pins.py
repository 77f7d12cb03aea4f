"""Pins of the oracle's Q/K normalisation and rotary embedding (CPU).

Doge guide, DMA forward step 1: Q and K pass through q_norm / k_norm (an
RMSNorm over head_dim with a per-element weight) and then the rotary position
embedding of the Llama code.  Each test checks the oracle against something
other than its own formula: the complex-number form of a rotation (numpy's
complex exponential), closed forms of RMSNorm, and invariants of rotary
embeddings (pair norms, dependence of dot products on relative position only).
"""
import numpy as np
import pytest

import oracle


def _rope_complex(y, pos, theta):
    """y rotated as complex pairs (y_e + i*y_{e+d/2}) * exp(i*pos*f_e), with
    the frequencies written as 1 / theta^(arange(0, d, 2) / d)."""
    d = y.shape[-1]
    freqs = 1.0 / theta ** (np.arange(0, d, 2, dtype=np.float64) / d)
    z = (y[..., : d // 2] + 1j * y[..., d // 2:]) * np.exp(1j * np.asarray(pos, np.float64)[..., None] * freqs)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("d", [8, 64, 128])
def test_rotation_is_complex_multiplication(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((5, d)).astype(np.float32)
    w = (0.5 + rng.random(d)).astype(np.float32)
    pos = np.array([0, 1, 7, 300, 4095])
    theta = 10000.0
    y = oracle.qk_norm_rope(x, w, 1e-6, theta, np.zeros(5, np.int32))   # position 0: normalisation only
    got = oracle.qk_norm_rope(x, w, 1e-6, theta, pos)
    assert np.allclose(got, _rope_complex(y, pos, theta), rtol=1e-12, atol=1e-12)


def test_unit_vector_pairs_with_the_second_half():
    # e_k turns in the (k, k + d/2) plane towards +e_{k+d/2}: the pairing and
    # the direction of the rotation
    d, theta = 16, 500.0
    for k in range(d // 2):
        x = np.zeros((1, d), np.float32)
        x[0, k] = 1.0
        got = oracle.qk_norm_rope(x, np.ones(d, np.float32), 0.0, theta, [9])[0]
        a = 9.0 / theta ** (2 * k / d)
        expect = np.zeros(d)
        expect[k] = np.sqrt(d) * np.cos(a)
        expect[k + d // 2] = np.sqrt(d) * np.sin(a)
        assert np.allclose(got, expect, atol=1e-12), k


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.3])
def test_rmsnorm_closed_form(eps):
    rng = np.random.default_rng(3)
    d = 64
    x = (rng.standard_normal((7, d)) * rng.uniform(0.01, 20, (7, 1))).astype(np.float32)
    y = oracle.qk_norm_rope(x, np.ones(d, np.float32), eps, 10000.0, np.zeros(7, np.int32))
    ms = (x.astype(np.float64) ** 2).mean(axis=1)
    # the root mean square of the output is sqrt(ms / (ms + eps))
    assert np.allclose(np.sqrt((y ** 2).mean(axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-12)
    # and the output points along x
    cos = (y * x).sum(1) / np.linalg.norm(y, axis=1) / np.linalg.norm(x.astype(np.float64), axis=1)
    assert np.allclose(cos, 1.0, atol=1e-12)


def test_rmsnorm_scale_invariance_and_weight():
    rng = np.random.default_rng(4)
    d = 32
    x = rng.standard_normal((3, d)).astype(np.float32)
    w = rng.standard_normal(d).astype(np.float32)
    a = oracle.qk_norm_rope(x, w, 0.0, 100.0, [5, 6, 7])
    b = oracle.qk_norm_rope((x * 4).astype(np.float32), w, 0.0, 100.0, [5, 6, 7])   # exact scaling in fp32
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    one = oracle.qk_norm_rope(x, np.ones(d, np.float32), 0.0, 100.0, np.zeros(3, np.int32))
    ww = oracle.qk_norm_rope(x, w, 0.0, 100.0, np.zeros(3, np.int32))
    assert np.allclose(ww, one * w, rtol=1e-12, atol=1e-14)


def test_pair_norms_kept_and_relative_position():
    rng = np.random.default_rng(5)
    d, theta = 64, 10000.0
    q = rng.standard_normal((1, d)).astype(np.float32)
    k = rng.standard_normal((1, d)).astype(np.float32)
    w = np.ones(d, np.float32)
    y0 = oracle.qk_norm_rope(q, w, 1e-6, theta, [0])[0]
    for p in (1, 33, 1000):
        y = oracle.qk_norm_rope(q, w, 1e-6, theta, [p])[0]
        assert np.allclose(y[: d // 2] ** 2 + y[d // 2:] ** 2, y0[: d // 2] ** 2 + y0[d // 2:] ** 2, rtol=1e-12)
    # <rope(q, m), rope(k, n)> depends on m - n only
    dots = []
    for m, n in ((10, 3), (110, 103), (2010, 2003)):
        dots.append(oracle.qk_norm_rope(q, w, 1e-6, theta, [m])[0] @ oracle.qk_norm_rope(k, w, 1e-6, theta, [n])[0])
    assert np.allclose(dots, dots[0], rtol=1e-9)


def test_bf16_inputs_read_exactly():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    w = rng.standard_normal(64).astype(np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    wb = (w.view(np.uint32) >> 16).astype(np.uint16)
    xt = (xb.astype(np.uint32) << 16).view(np.float32)
    wt = (wb.astype(np.uint32) << 16).view(np.float32)
    a = oracle.qk_norm_rope(xb, wb, 1e-6, 10000.0, [1, 2, 3, 4])
    b = oracle.qk_norm_rope(xt, wt, 1e-6, 10000.0, [1, 2, 3, 4])
    assert np.array_equal(a, b)

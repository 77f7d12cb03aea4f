"""GPU parity of the CDMoE routed experts against the oracle.

Bars: routing from the same float32 logits is bit-exact in the expert lists
(the decision is taken on float32 pair sums on both sides) and the weights
within 1e-5 relative; logits (float32 accumulation of exact bf16 products
over H terms) within 1e-5 of the row's largest |logit| plus 1e-6; expert
outputs (float32 arithmetic, one bf16 rounding) within half a bf16 ulp plus
1e-5 of the largest output.
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


@pytest.mark.parametrize("T,nk,k,kind", [(100, 128, 64, "normal"), (37, 16, 16, "normal"), (50, 12, 5, "few"),
                                         (20, 256, 128, "normal"), (9, 1, 1, "normal"), (64, 128, 64, "few")])
def test_route_bit_exact(dma, oracle_mod, T, nk, k, kind):
    rng = np.random.default_rng(T + nk + k)
    if kind == "few":
        logits = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(T, 2 * nk))
    else:
        logits = rng.standard_normal((T, 2 * nk)).astype(np.float32)
    idx, w = dma.cdmoe_route(to_dev(logits), k)
    torch.cuda.synchronize()
    ri, rw = oracle_mod.cdmoe_route(logits, k)
    np.testing.assert_array_equal(to_host(idx), ri)
    assert np.allclose(to_host(w), rw, rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("T,H,nk", [(130, 1024, 128), (7, 512, 16), (64, 1536, 5)])
def test_logits(dma, oracle_mod, T, H, nk):
    h, router, _, _ = si.make_cdmoe(T, H, 1, "bf16", seed=T)
    router = si.make_cdmoe(1, H, nk, "bf16", seed=T + 1)[1]
    got = to_host(dma.cdmoe_logits(to_dev(h), to_dev(router)))
    ref = oracle_mod.cdmoe_logits(h, router)
    bound = 1e-5 * np.abs(ref).max(axis=1, keepdims=True) + 1e-6
    assert (np.abs(got - ref) <= bound).all(), np.abs(got - ref).max()


@pytest.mark.parametrize("T,H,nk,k", [(40, 1024, 128, 64), (9, 512, 8, 64), (33, 1536, 16, 1)])
def test_experts(dma, oracle_mod, T, H, nk, k):
    h, _, down, up = si.make_cdmoe(T, H, nk, "bf16", seed=H + k)
    rng = np.random.default_rng(k)
    idx = rng.integers(0, nk * nk, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    got = to_host(dma.cdmoe_experts(to_dev(h), to_dev(down), to_dev(up), to_dev(idx), to_dev(w)))
    ref = oracle_mod.cdmoe_experts(h, down, up, idx, w.astype(np.float64))
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max()
    assert (np.abs(got - ref) <= bound).all(), np.abs(got - ref).max()


def test_chain_at_config_size(dma, oracle_mod):
    """logits -> route -> experts at the DogeConfig sizes (hidden 1024,
    16384 experts, 64 per token) against the whole fp64 oracle.
    The routing decision is taken in float32 on both sides: the oracle's
    routing of the GPU's float32 logits must give the GPU's expert lists
    for every token.  Against the fp64 chain, a token's list may differ only
    where the fp64 pair scores leave no float32-resolvable gap at the k-th
    place: its k-th and (k+1)-th best pair scores (over all nk*nk pairs) lie
    within twice the token's largest logit error plus float32 rounding, and
    every expert in only one of the two lists scores within that margin of
    the k-th.  Every token whose list agrees is output-checked."""
    T, H, nk, k = 256, 1024, 128, 64
    h, router, down, up = si.make_cdmoe(T, H, nk, "bf16", seed=12)
    hd = to_dev(h)
    lg = dma.cdmoe_logits(hd, to_dev(router))
    idx, w = dma.cdmoe_route(lg, k)
    out = dma.cdmoe_experts(hd, to_dev(down), to_dev(up), idx, w)
    torch.cuda.synchronize()
    gl, gi, go = to_host(lg), to_host(idx), to_host(out)
    # the decision in the kernel's precision: exact for every token
    fi, _ = oracle_mod.cdmoe_route(gl, k)
    np.testing.assert_array_equal(gi, fi)
    # against the fp64 chain
    ri, rw, ro = oracle_mod.cdmoe(h, router, down, up, k)
    rl = oracle_mod.cdmoe_logits(h, router)
    same = (gi == ri).all(axis=1)
    for t in np.nonzero(~same)[0]:
        x, y = rl[t, :nk], rl[t, nk:]
        scores = (x[:, None] + y[None, :]).ravel()          # expert a*nk + b scores x_a + y_b
        srt = np.sort(scores)[::-1]
        err = np.abs(gl[t].astype(np.float64) - rl[t]).max()
        margin = 2.0 * err + 4.0 * np.spacing(np.float32(abs(srt[k - 1])))
        assert srt[k - 1] - srt[k] <= margin, (t, srt[k - 1] - srt[k], margin)
        diff = np.setxor1d(gi[t], ri[t])
        assert (np.abs(scores[diff] - srt[k - 1]) <= margin).all(), (t, diff)
    assert same.sum() > 0
    bound = 2.0 ** -8 * np.abs(ro[same]) + 1e-4 * np.abs(ro).max()
    assert (np.abs(go[same] - ro[same]) <= bound).all()

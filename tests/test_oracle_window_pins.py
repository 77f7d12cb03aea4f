"""Pins of the oracle's sliding-window variant (CPU).

DogeConfig's sliding_window makes the attention mask the sliding-window causal
mask (row i sees keys i - win < j <= i); the dynamic mask then keeps the top
keep_window_size of the visible keys.  The oracle (row_kept with a window) is
checked against: the literal NumPy brute force (tests/brute.py), which
materialises the min_dtype mask with the window and sorts whole rows; the
full-causal oracle when the window covers the sequence; and the library SDPA
routine with a float mask when the window is no wider than w (every visible
key is kept).
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests import brute


@pytest.mark.parametrize("S", [1, 9, 40, 97])
@pytest.mark.parametrize("kind", ["lognormal", "dyadic", "few", "const"])
def test_window_kept_sets_and_thresholds_match_brute(oracle_mod, S, kind):
    B, Hkv = 2, 2
    dt = si.make_dt((B, Hkv, S), kind, seed=S * 3 + len(kind))
    for seq in (None, np.array([S, max(1, S // 2)], np.int32)):
        for w, win in ((1, 3), (3, 1), (4, 9), (9, 4), (5, 5), (7, 20), (16, 33), (2, S + 4)):
            want = brute.kept_sets(dt, w, seq, win)
            tau, tie = oracle_mod.select(dt, w, seq, win=win)
            for b in range(B):
                L = S if seq is None else int(seq[b])
                for g in range(Hkv):
                    for i in range(S):
                        got = oracle_mod.kept_row(dt, w, b, g, i, seq, win=win)
                        exp = np.flatnonzero(want[b, g, i]) if i < L else np.array([], int)
                        assert got.tolist() == exp.tolist(), (b, g, i, w, win)
                        visible = min(i, L - 1) - max(0, i - win + 1) + 1
                        if i >= L:
                            assert tau[b, g, i] == np.inf and tie[b, g, i] == -1
                        elif visible <= w:
                            assert tau[b, g, i] == -np.inf and tie[b, g, i] == -1
                        else:
                            last = sorted(exp.tolist(), key=lambda k: (-float(dt[b, g, k]), k))[-1]
                            assert tie[b, g, i] == last and tau[b, g, i] == dt[b, g, last]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_window_attention_matches_brute(oracle_mod, dtype):
    B, S, Hq, Hkv, d = 2, 37, 4, 2, 16
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, dtype, 5)
    dt = si.make_dt((B, Hkv, S), "few", 6)
    seq = np.array([37, 20], np.int32)
    f = (lambda x: si.bf16_bits_to_f32(x)) if dtype == "bf16" else (lambda x: x)
    for w, win in ((3, 8), (8, 3), (6, 6), (10, 50)):
        got = oracle_mod.attn(Q, K, V, dt, w, seq, win=win)
        ref = brute.attention(f(Q), f(K), f(V), dt, w, seq, win)
        for b in range(B):
            assert np.allclose(got[b, :seq[b]], ref[b, :seq[b]], rtol=1e-12, atol=1e-12), (w, win)
            assert not got[b, seq[b]:].any()


def test_wide_window_is_full_causal(oracle_mod):
    B, S, Hq, Hkv, d, w = 2, 64, 4, 2, 16, 11
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "f32", 7)
    dt = si.make_dt((B, Hkv, S), "dyadic", 8)
    seq = np.array([64, 30], np.int32)
    for win in (S, S + 1, 10 * S):
        a = oracle_mod.select(dt, w, seq, win=win)
        b = oracle_mod.select(dt, w, seq)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert np.array_equal(oracle_mod.attn(Q, K, V, dt, w, seq, win=win), oracle_mod.attn(Q, K, V, dt, w, seq))


def test_narrow_window_is_sliding_window_sdpa(oracle_mod):
    """win <= w: every visible key is kept, so the result is sliding-window
    causal attention with the dt bias (the library's SDPA with a float mask)."""
    B, S, Hq, Hkv, d = 1, 50, 2, 1, 32
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, "f32", 9)
    dt = si.make_dt((B, Hkv, S), "lognormal", 10)
    for w, win in ((8, 8), (20, 5), (3, 1)):
        got = oracle_mod.attn(Q, K, V, dt, w, win=win)
        i = np.arange(S)[:, None]
        j = np.arange(S)[None, :]
        vis = (j <= i) & (j > i - win)
        m = np.where(vis, dt[0, 0][None, :].astype(np.float64), -np.inf)
        q = torch.tensor(Q[0].transpose(1, 0, 2), dtype=torch.float64)      # [Hq, S, d]
        k = torch.tensor(K[0].transpose(1, 0, 2), dtype=torch.float64).expand(Hq, S, d)
        v = torch.tensor(V[0].transpose(1, 0, 2), dtype=torch.float64).expand(Hq, S, d)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.tensor(m))
        assert np.allclose(got[0], ref.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12), (w, win)

"""The C oracle against the literal NumPy brute force (tests/brute.py) on tiny shapes.

The brute force materialises the min_dtype mask and sorts whole rows, the way
the gitcode Doge guide's DMA section describes the procedure; the oracle
selects per row over valid keys only.  Agreement pins both the selection and
the attention of the oracle, including padding, ties, and every edge case of w.
"""
import numpy as np
import pytest

import synth_inputs as si
from tests import brute

SHAPES = [1, 2, 17, 64, 130]


def _ws(S):
    return sorted({1, 2, 7, 64, max(S - 1, 1), S, S + 5})


@pytest.mark.parametrize("S", SHAPES)
@pytest.mark.parametrize("kind", ["lognormal", "dyadic", "few", "const"])
def test_kept_sets_match_brute(oracle_mod, S, kind):
    B, Hkv = 2, 2
    dt = si.make_dt((B, Hkv, S), kind, seed=S * 7 + len(kind))
    for seq in (None, np.array([S, max(1, S // 2)], np.int32)):
        for w in _ws(S):
            want = brute.kept_sets(dt, w, seq)
            tau, tie = oracle_mod.select(dt, w, seq)
            for b in range(B):
                L = S if seq is None else int(seq[b])
                for g in range(Hkv):
                    for i in range(S):
                        got = oracle_mod.kept_row(dt, w, b, g, i, seq)
                        exp = np.flatnonzero(want[b, g, i]) if i < L else np.array([], int)
                        assert got.tolist() == exp.tolist(), (b, g, i, w)
                        if i < L and i + 1 > w:
                            # (tau, tie) is the last kept key in selection order
                            j = exp
                            order = sorted(j.tolist(), key=lambda k: (-float(dt[b, g, k]), k))
                            assert tie[b, g, i] == order[-1]
                            assert tau[b, g, i] == dt[b, g, order[-1]]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,w", [(1, 1), (17, 4), (64, 64), (64, 70), (130, 7), (130, 129)])
def test_attn_matches_brute(oracle_mod, dtype, S, w):
    B, Hq, Hkv, d = 2, 4, 2, 16
    Q, K, V = si.make_qkv(B, S, Hq, Hkv, d, dtype, seed=S + w)
    dt = si.make_dt((B, Hkv, S), "dyadic" if w % 2 else "lognormal", seed=w)
    seq = np.array([S, max(1, (2 * S) // 3)], np.int32)

    def f(x):
        return si.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x

    ref = brute.attention(f(Q), f(K), f(V), dt, w, seq)
    out = oracle_mod.attn(Q, K, V, dt, w, seqlens=seq)
    for b in range(B):
        L = int(seq[b])
        np.testing.assert_allclose(out[b, :L], ref[b, :L], rtol=0, atol=1e-12)
        assert (out[b, L:] == 0).all()

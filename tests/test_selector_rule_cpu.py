"""The decomposition the GPU selector relies on, checked against the oracle on the CPU.

For a chunk of C query rows starting at r0, each row's w-th kept key lies in
the band of prefix ranks [w-C-1, w) plus the chunk's own keys, and it is the
(w - A0)-th of those (in selection order) with index <= i, where
A0 = clamp(w-C-1, 0, r0).  This restates the claim in plain Python (sorting
with the selection order) and compares every row with the oracle.
"""
import numpy as np
import pytest

import synth_inputs as si


def band_rule(row, L, w, C):
    S = len(row)
    tau = np.empty(S, np.float32)
    tie = np.empty(S, np.int32)
    key = lambda j: (-float(row[j]), j)  # noqa: E731
    for r0 in range(0, S, C):
        rend, lo, hi = min(r0 + C, S), max(r0, w), min(r0 + C, L)
        for i in range(r0, rend):
            if i >= L:
                tau[i], tie[i] = np.inf, -1
            elif i < w:
                tau[i], tie[i] = -np.inf, -1
        if lo >= hi:
            continue
        A0 = max(0, min(r0, w - C - 1))
        band = sorted(range(r0), key=key)[A0:min(r0, w)]
        assert len(band) <= C + 1
        cand = sorted(band + list(range(r0, hi)), key=key)
        for i in range(lo, hi):
            eligible = [j for j in cand if j <= i]
            j = eligible[w - A0 - 1]
            tau[i], tie[i] = row[j], j
    return tau, tie


@pytest.mark.parametrize("trial", range(24))
def test_band_rule_matches_oracle(oracle_mod, trial):
    rng = np.random.default_rng(trial)
    S = int(rng.integers(1, 600))
    w = int(rng.integers(1, 700))
    C = [64, 16, 7][trial % 3]
    kind = ["dyadic", "few", "const", "lognormal"][trial % 4]
    dt = si.make_dt((1, 1, S), kind, seed=trial)
    L = int(rng.integers(1, S + 1))
    tau, tie = band_rule(dt[0, 0], L, w, C)
    rt, ri = oracle_mod.select(dt, w, np.array([L], np.int32))
    np.testing.assert_array_equal(tie, ri[0, 0])
    np.testing.assert_array_equal(tau, rt[0, 0])


def test_band_of_width_C_is_not_enough(oracle_mod):
    # With a band of only C prefix keys the rule misses rows whose C new keys
    # all beat the prefix key of rank w-C-1 (here row 703 for w=700, C=64).
    dt = si.make_dt((1, 1, 3000), "dyadic", seed=5)
    row = dt[0, 0]
    rt, ri = oracle_mod.select(dt, 700)
    r0, C, w = 640, 64, 700
    key = lambda j: (-float(row[j]), j)  # noqa: E731
    band_c = sorted(range(r0), key=key)[w - C:w]
    cand = sorted(band_c + list(range(r0, r0 + C)), key=key)
    wrong = [j for j in cand if j <= 703][C - 1]
    assert wrong != ri[0, 0, 703]
    tau, tie = band_rule(row, 3000, w, C)
    assert tie[703] == ri[0, 0, 703]

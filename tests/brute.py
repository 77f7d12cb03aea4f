"""Literal brute force of the Doge guide's mask procedure, NumPy fp64, tiny shapes only.

Independent of the C oracle (no shared code).  It follows the gitcode Doge guide,
section on Dynamic Mask Attention, forward step 3 as written: the per-key dt is
broadcast to a full [batch, kv_heads, query_len, key_len] tensor, causal and
padding positions are filled with min_dtype (the most negative float32), and --
only when the key length exceeds keep_window_size -- each row keeps its
keep_window_size largest entries (a stable sort, so among equal values the
lower key index comes first) and the rest become min_dtype.  Step 4: the mask
is added to the head_dim**-0.5 scaled scores of each query head (query head hq
reads kv head hq // G) and a softmax in fp64 gives the weights of V.
"""
from __future__ import annotations

import numpy as np

MIN_DTYPE = float(np.finfo(np.float32).min)


def mask(dt32, w, seqlens=None, win=None):
    """Materialised additive mask M[b, g, i, j] (float64).  win: the sliding-window
    causal mask of DogeConfig's sliding_window (row i sees i - win < j <= i)."""
    dt32 = np.asarray(dt32, dtype=np.float32)
    B, Hkv, S = dt32.shape
    M = np.broadcast_to(dt32[:, :, None, :].astype(np.float64), (B, Hkv, S, S)).copy()
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    M[:, :, j > i] = MIN_DTYPE
    if win is not None:
        M[:, :, j <= i - win] = MIN_DTYPE
    if seqlens is not None:
        for b in range(B):
            M[b, :, :, int(seqlens[b]):] = MIN_DTYPE
    if S > w:
        order = np.argsort(-M, axis=-1, kind="stable")
        keep = np.zeros(M.shape, dtype=bool)
        np.put_along_axis(keep, order[..., :w], True, axis=-1)
        M = np.where(keep, M, MIN_DTYPE)
    return M


def kept_sets(dt32, w, seqlens=None, win=None):
    """Boolean [B,Hkv,S,S]: key j takes part in row i's softmax."""
    return mask(dt32, w, seqlens, win) > MIN_DTYPE


def attention(Q, K, V, dt32, w, seqlens=None, win=None):
    """fp64 output [B,S,Hq,d] of the masked softmax; Q/K/V given as float arrays."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    M = mask(dt32, w, seqlens, win)
    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        for hq in range(Hq):
            g = hq // G
            s = (Q[b, :, hq, :] @ K[b, :, g, :].T) / np.sqrt(d) + M[b, g]
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=-1, keepdims=True)
            out[b, :, hq, :] = p @ V[b, :, g, :]
    return out

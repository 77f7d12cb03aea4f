"""CPU oracle for the DMA forward hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``libdma.so`` and the
``doge_dynamic_mask_amd`` binding) never imports, links or calls it, and the two
share no code: the oracle is plain C in fp64 (``dma_oracle.c``) plus these
ctypes wrappers, which only marshal NumPy arrays.

Each function follows the gitcode "Doge guide" page, section on Dynamic Mask
Attention (forward chain steps 3 and 4); the C source cites the step for every
function.  Pins live in ``tests/test_oracle_pins.py`` and
``tests/test_oracle_vs_brute.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dma_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1


def build(force: bool = True) -> str:
    """Compile ``dma_oracle.c`` into ``liboracle.so`` with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        lib.oracle_dt.argtypes = [P, P, P, P, I, I, I, I, I, P]
        lib.oracle_dt.restype = None
        lib.oracle_select.argtypes = [P, P, I, I, I, I, I, P, I64, P, P]
        lib.oracle_select.restype = None
        lib.oracle_kept_row.argtypes = [P, P, I, I, I, I, I, I, I, P]
        lib.oracle_kept_row.restype = ctypes.c_int
        lib.oracle_attn.argtypes = [P, P, P, I, P, P, I, I, I, I, I, I, I, P, I64, P]
        lib.oracle_attn.restype = None
        lib.oracle_decode.argtypes = [P, P, P, I, P, P, I, I, I, I, I, I, P, P]
        lib.oracle_decode.restype = None
        lib.oracle_qk_norm_rope.argtypes = [P, P, I, ctypes.c_double, ctypes.c_double, P, I64, I, P]
        lib.oracle_qk_norm_rope.restype = None
        lib.oracle_attn_bwd.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I, I, P, P, P, P]
        lib.oracle_attn_bwd.restype = None
        lib.oracle_dt_bwd.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P, P, P]
        lib.oracle_dt_bwd.restype = None
        lib.oracle_cdmoe.argtypes = [P, P, P, P, I, I, I, I, I, P, P, P]
        lib.oracle_cdmoe.restype = None
        lib.oracle_cdmoe_route.argtypes = [P, I, I, I, P, P]
        lib.oracle_cdmoe_route.restype = None
        lib.oracle_cdmoe_logits.argtypes = [P, P, I, I, I, I, P]
        lib.oracle_cdmoe_logits.restype = None
        lib.oracle_cdmoe_experts.argtypes = [P, P, P, I, P, P, I, I, I, P]
        lib.oracle_cdmoe_experts.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _elem_array(x):
    """float32 arrays pass as F32; uint16 arrays hold bfloat16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle inputs are float32 or bf16 bits (uint16), got {x.dtype}")


def _rows_array(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    return r, r.shape[0]


def _seq(seqlens):
    return None if seqlens is None else np.ascontiguousarray(seqlens, dtype=np.int32)


def dt(V, W, bias, A):
    """dt in fp64, [B, Hkv, S], from V [B,S,Hkv,d], W [Hkv,Hkv*d], bias [Hkv]|None, A [Hkv]."""
    V, tv = _elem_array(V)
    W, tw = _elem_array(W)
    assert tv == tw
    if bias is not None:
        bias, tb = _elem_array(bias)
        assert tb == tv
    A = np.ascontiguousarray(A, dtype=np.float32)
    B, S, Hkv, d = V.shape
    assert W.shape == (Hkv, Hkv * d) and A.shape == (Hkv,)
    out = np.empty((B, Hkv, S), dtype=np.float64)
    _load().oracle_dt(_ptr(V), _ptr(W), _ptr(bias), _ptr(A), tv, B, S, Hkv, d, _ptr(out))
    return out


def select(dt32, w, seqlens=None, rows=None, win=None):
    """(tau, tie) per row.  dt32 is float32 [B,Hkv,S]; rows is an optional (n,3) list of (b,g,i);
    win: sliding window of win positions (None: full causal)."""
    dt32 = np.ascontiguousarray(dt32, dtype=np.float32)
    B, Hkv, S = dt32.shape
    r, n = _rows_array(rows)
    shape = (n,) if r is not None else (B, Hkv, S)
    tau = np.empty(shape, dtype=np.float32)
    tie = np.empty(shape, dtype=np.int32)
    seq = _seq(seqlens)
    _load().oracle_select(_ptr(dt32), _ptr(seq), B, Hkv, S, int(w), int(win or 0), _ptr(r), n, _ptr(tau), _ptr(tie))
    return tau, tie


def kept_row(dt32, w, b, g, i, seqlens=None, win=None):
    """Kept key indices of one row, ascending (win: sliding window, None for full causal)."""
    dt32 = np.ascontiguousarray(dt32, dtype=np.float32)
    B, Hkv, S = dt32.shape
    out = np.empty(max(int(w), 1), dtype=np.int32)
    seq = _seq(seqlens)
    n = _load().oracle_kept_row(_ptr(dt32), _ptr(seq), Hkv, S, int(w), int(win or 0), int(b), int(g), int(i),
                                _ptr(out))
    return out[:n].copy()


def attn(Q, K, V, dt32, w, seqlens=None, rows=None, win=None):
    """fp64 attention.  Full [B,S,Hq,d] output, or [n, G, d] for a (b,g,i) row list.
    win: sliding window of win positions (None: full causal)."""
    Q, tq = _elem_array(Q)
    K, tk = _elem_array(K)
    V, tv = _elem_array(V)
    assert tq == tk == tv
    dt32 = np.ascontiguousarray(dt32, dtype=np.float32)
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    assert K.shape == (B, S, Hkv, d) and V.shape == K.shape and Hq % Hkv == 0
    assert dt32.shape == (B, Hkv, S)
    G = Hq // Hkv
    r, n = _rows_array(rows)
    out = np.empty((n, G, d) if r is not None else (B, S, Hq, d), dtype=np.float64)
    seq = _seq(seqlens)
    _load().oracle_attn(_ptr(Q), _ptr(K), _ptr(V), tq, _ptr(dt32), _ptr(seq), B, S, Hq, Hkv, d,
                        int(w), int(win or 0), _ptr(r), n, _ptr(out))
    return out


def decode(q, Kc, Vc, dt_cache, cache_lens, w):
    """fp64 decode output [B,Hq,d] and kept indices [B,Hkv,w] (ascending, -1 padded)."""
    q, tq = _elem_array(q)
    Kc, tk = _elem_array(Kc)
    Vc, tv = _elem_array(Vc)
    assert tq == tk == tv
    B, Hq, d = q.shape
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    dt_cache = np.ascontiguousarray(dt_cache, dtype=np.float32)
    assert dt_cache.shape == (B, Hkv, Lmax)
    lens = np.ascontiguousarray(cache_lens, dtype=np.int32)
    out = np.empty((B, Hq, d), dtype=np.float64)
    kept = np.empty((B, Hkv, int(w)), dtype=np.int32)
    _load().oracle_decode(_ptr(q), _ptr(Kc), _ptr(Vc), tq, _ptr(dt_cache), _ptr(lens), B, Lmax, Hq,
                          Hkv, d, int(w), _ptr(out), _ptr(kept))
    return out, kept


def qk_norm_rope(x, w, eps, theta, positions):
    """RMSNorm over the last axis (weight w) then the rotary embedding, fp64.

    x: [..., d] (float32 or bf16 bit patterns), w: [d] of the same type,
    positions: int array broadcastable to x.shape[:-1] (the position of each
    row).  Doge guide, DMA forward step 1 (q_norm / k_norm, rotary)."""
    x, tx = _elem_array(x)
    w, tw = _elem_array(w)
    assert tx == tw
    d = x.shape[-1]
    assert w.shape == (d,) and d % 2 == 0
    pos = np.ascontiguousarray(np.broadcast_to(np.asarray(positions, np.int32), x.shape[:-1]), dtype=np.int32)
    n = int(np.prod(x.shape[:-1]))
    out = np.empty(x.shape, dtype=np.float64)
    _load().oracle_qk_norm_rope(_ptr(x), _ptr(w), tx, float(eps), float(theta), _ptr(pos), n, d, _ptr(out))
    return out


def attn_bwd(Q, K, V, dt32, w, dO, seqlens=None):
    """fp64 gradients (dQ, dK, dV, ddt) of attn() for an upstream gradient dO [B,S,Hq,d]
    (same storage type as Q).  Kept sets are the forward's; selection has no gradient."""
    Q, tq = _elem_array(Q)
    K, tk = _elem_array(K)
    V, tv = _elem_array(V)
    dO, to = _elem_array(dO)
    assert tq == tk == tv == to
    dt32 = np.ascontiguousarray(dt32, dtype=np.float32)
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    assert K.shape == (B, S, Hkv, d) and V.shape == K.shape and dO.shape == Q.shape and Hq % Hkv == 0
    assert dt32.shape == (B, Hkv, S)
    dQ = np.empty((B, S, Hq, d))
    dK = np.empty((B, S, Hkv, d))
    dV = np.empty((B, S, Hkv, d))
    ddt = np.empty((B, Hkv, S))
    seq = _seq(seqlens)
    _load().oracle_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), tq, _ptr(dt32), _ptr(seq), _ptr(dO), B, S, Hq, Hkv, d,
                            int(w), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ddt))
    return dQ, dK, dV, ddt


def dt_bwd(V, W, bias, A, ddt):
    """fp64 gradients of dt() for an upstream gradient ddt [B,Hkv,S]:
    (dV through dt_proj [B,S,Hkv,d], dW [Hkv,Hkv*d], dbias [Hkv], dA [Hkv])."""
    V, tv = _elem_array(V)
    W, tw = _elem_array(W)
    assert tv == tw
    if bias is not None:
        bias, tb = _elem_array(bias)
        assert tb == tv
    A = np.ascontiguousarray(A, dtype=np.float32)
    B, S, Hkv, d = V.shape
    assert W.shape == (Hkv, Hkv * d) and A.shape == (Hkv,)
    ddt = np.ascontiguousarray(ddt, dtype=np.float64)
    assert ddt.shape == (B, Hkv, S)
    dV = np.empty((B, S, Hkv, d))
    dW = np.empty((Hkv, Hkv * d))
    dbias = np.empty(Hkv)
    dA = np.empty(Hkv)
    _load().oracle_dt_bwd(_ptr(V), _ptr(W), _ptr(bias), _ptr(A), tv, B, S, Hkv, d, _ptr(ddt), _ptr(dV), _ptr(dW),
                          _ptr(dbias), _ptr(dA))
    return dV, dW, dbias, dA


def cdmoe(h, router, down, up, k):
    """CDMoE routed experts, fp64: (idx [T,k] int32 in selection order, weights [T,k], out [T,H]).
    h [T,H], router [2*nk,H], down/up [nk*nk,H], all float32 or all bf16 bits."""
    h, th = _elem_array(h)
    router, tr = _elem_array(router)
    down, td = _elem_array(down)
    up, tu = _elem_array(up)
    assert th == tr == td == tu
    T, H = h.shape
    nk = router.shape[0] // 2
    assert router.shape == (2 * nk, H) and down.shape == (nk * nk, H) and up.shape == down.shape and k <= nk
    idx = np.empty((T, k), np.int32)
    wts = np.empty((T, k))
    out = np.empty((T, H))
    _load().oracle_cdmoe(_ptr(h), _ptr(router), _ptr(down), _ptr(up), th, T, H, nk, int(k), _ptr(idx), _ptr(wts),
                         _ptr(out))
    return idx, wts, out


def cdmoe_route(logits, k):
    """Routing from float32 logits [T, 2*nk]: (idx [T,k] int32 in selection order, weights [T,k])."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, n2 = logits.shape
    nk = n2 // 2
    assert k <= nk
    idx = np.empty((T, k), np.int32)
    wts = np.empty((T, k))
    _load().oracle_cdmoe_route(_ptr(logits), T, nk, int(k), _ptr(idx), _ptr(wts))
    return idx, wts


def cdmoe_logits(h, router):
    """Router logits [T, 2*nk] in fp64."""
    h, th = _elem_array(h)
    router, tr = _elem_array(router)
    assert th == tr
    T, H = h.shape
    nk = router.shape[0] // 2
    out = np.empty((T, 2 * nk))
    _load().oracle_cdmoe_logits(_ptr(h), _ptr(router), th, T, H, nk, _ptr(out))
    return out


def cdmoe_experts(h, down, up, idx, wts):
    """Expert output [T, H] in fp64 for given kept experts idx [T, k] and weights [T, k]."""
    h, th = _elem_array(h)
    down, td = _elem_array(down)
    up, tu = _elem_array(up)
    assert th == td == tu
    T, H = h.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    wts = np.ascontiguousarray(wts, dtype=np.float64)
    k = idx.shape[1]
    out = np.empty((T, H))
    _load().oracle_cdmoe_experts(_ptr(h), _ptr(down), _ptr(up), th, _ptr(idx), _ptr(wts), T, H, k, _ptr(out))
    return out

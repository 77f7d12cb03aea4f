"""Python binding of libdma.so, the MI355X forward hot path of Doge's Dynamic Mask Attention.

Thin ctypes marshalling only: every step runs in the HIP kernels of
``libdma.so``.  torch supplies device memory (outputs and workspace are
allocated with torch on the inputs' device) and the current stream.  There is
no CPU fallback: if the library is missing, importing the binding's functions
raises.

Functions mirror the C ABI in ``include/dma.h``:

    dt(V, W, A, bias=None, out=None, out_pos=None)      -> dt [B, Hkv, S] float32
    select(dt, w, seqlens=None)                         -> (tau, tie)
    attn_fwd(Q, K, V, dt, tau, tie, w, seqlens=None)    -> O
    decode(q, Kc, Vc, dt_cache, cache_lens, w, kept=False) -> out (, kept_idx)
    prefill(Q, K, V, W, A, w, bias=None, seqlens=None)  -> (O, dt, tau, tie)
    qk_norm_rope(Q, K, q_norm_w, k_norm_w, ...)         -> (Q', K')
    prologue(Q, K, V, q_norm_w, k_norm_w, W, A, ...)    -> (Q', K', dt)
    DecodeState, decode_state_init(...), decode_step(...)  incremental decode
    attn_bwd(Q, K, V, dt, tau, tie, w, dO, seqlens=None) -> (dQ, dK, dV, ddt)
    dt_bwd(V, W, A, ddt, bias=None, dV=None)            -> (dW, dbias, dA); adds into dV
    prefill_bwd(Q, K, V, W, A, w, dO, ...)               -> dict of every gradient
    select_window(dt, w, win, seqlens=None)             -> (tau, tie) under a sliding window
    attn_window_fwd(Q, K, V, dt, tau, tie, w, win, seqlens=None) -> O
    cdmoe_logits(h, router), cdmoe_route(logits, k), cdmoe_experts(h, down, up, idx, weights)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdma.so")

F32 = 0
BF16 = 1

_STATUS = {
    0: "DMA_OK", -1: "DMA_ERR_NULL", -2: "DMA_ERR_SHAPE", -3: "DMA_ERR_DTYPE",
    -4: "DMA_ERR_UNSUPPORTED", -5: "DMA_ERR_WORKSPACE", -6: "DMA_ERR_HIP",
}

EXPORTS = ("dma_version", "dma_status_str", "dma_workspace_bytes", "dma_dt", "dma_select", "dma_attn_fwd",
           "dma_decode_workspace_bytes", "dma_decode", "dma_decode_noalloc", "dma_decode_state_bytes",
           "dma_decode_step_workspace_bytes", "dma_decode_state_init", "dma_decode_step",
           "dma_decode_state_kept", "dma_qk_norm_rope", "dma_prologue",
           "dma_attn_bwd_workspace_bytes", "dma_attn_bwd", "dma_dt_bwd_workspace_bytes", "dma_dt_bwd",
           "dma_select_window", "dma_attn_window_fwd", "dma_cdmoe_logits", "dma_cdmoe_route",
           "dma_cdmoe_experts")


class DmaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_STATUS.get(status, status)} ({lib().dma_status_str(status).decode()})")


_lib = None


def lib():
    """The loaded libdma.so (ctypes.CDLL) with argument types set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m doge_dynamic_mask_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    L.dma_version.argtypes, L.dma_version.restype = [], I
    L.dma_status_str.argtypes, L.dma_status_str.restype = [I], ctypes.c_char_p
    L.dma_workspace_bytes.argtypes, L.dma_workspace_bytes.restype = [I, I, I, I, I, I, I], SZ
    L.dma_dt.argtypes = [P, P, P, P, I, I, I, I, I, P, I64, P, P]
    L.dma_dt.restype = I
    L.dma_select.argtypes = [P, P, I, I, I, I, P, P, P]
    L.dma_select.restype = I
    L.dma_attn_fwd.argtypes = [P, P, P, I, P, P, P, P, I, I, I, I, I, I, P, P]
    L.dma_attn_fwd.restype = I
    L.dma_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.dma_decode_workspace_bytes.restype = SZ
    L.dma_decode.argtypes = [P, P, P, I, P, P, I, I, I, I, I, I, P, P, P, SZ, P]
    L.dma_decode.restype = I
    L.dma_decode_noalloc.argtypes = [P, P, P, I, P, P, I, I, I, I, I, I, P, P, P]
    L.dma_decode_noalloc.restype = I
    L.dma_decode_state_bytes.argtypes, L.dma_decode_state_bytes.restype = [I, I, I, I], SZ
    L.dma_decode_step_workspace_bytes.argtypes = [I, I, I, I, I]
    L.dma_decode_step_workspace_bytes.restype = SZ
    L.dma_decode_state_init.argtypes = [P, P, I, P, P, I, I, I, I, I, P, SZ, P, SZ, P]
    L.dma_decode_state_init.restype = I
    L.dma_decode_step.argtypes = [P, P, P, I, P, I, I, I, I, I, P, SZ, P, P, SZ, P]
    L.dma_decode_step.restype = I
    L.dma_decode_state_kept.argtypes = [P, SZ, I, I, I, I, P, P, P]
    L.dma_decode_state_kept.restype = I
    D = ctypes.c_double
    L.dma_qk_norm_rope.argtypes = [P, P, I, P, P, ctypes.c_float, D, P, I, I, I, I, I, P, P, P]
    L.dma_qk_norm_rope.restype = I
    L.dma_prologue.argtypes = [P, P, P, I, P, P, ctypes.c_float, D, P, P, P, P, I, I, I, I, I, P, P, P, P]
    L.dma_prologue.restype = I
    L.dma_attn_bwd_workspace_bytes.argtypes = [I, I, I, I, I, I]
    L.dma_attn_bwd_workspace_bytes.restype = SZ
    L.dma_attn_bwd.argtypes = [P, P, P, I, P, P, P, P, P, I, I, I, I, I, I, P, P, P, P, P, SZ, P]
    L.dma_attn_bwd.restype = I
    L.dma_dt_bwd_workspace_bytes.argtypes = [I, I, I, I]
    L.dma_dt_bwd_workspace_bytes.restype = SZ
    L.dma_dt_bwd.argtypes = [P, P, P, P, I, P, I, I, I, I, P, P, P, P, P, SZ, P]
    L.dma_dt_bwd.restype = I
    L.dma_select_window.argtypes = [P, P, I, I, I, I, I, P, P, P]
    L.dma_select_window.restype = I
    L.dma_attn_window_fwd.argtypes = [P, P, P, I, P, P, P, P, I, I, I, I, I, I, I, P, P]
    L.dma_attn_window_fwd.restype = I
    L.dma_cdmoe_logits.argtypes = [P, P, I, I, I, I, P, P]
    L.dma_cdmoe_logits.restype = I
    L.dma_cdmoe_route.argtypes = [P, I, I, I, P, P, P]
    L.dma_cdmoe_route.restype = I
    L.dma_cdmoe_experts.argtypes = [P, P, P, I, P, P, I, I, I, I, P, P]
    L.dma_cdmoe_experts.restype = I
    _lib = L
    return L


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"expected bfloat16 or float32, got {t.dtype}")


def _check(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(ws, nbytes, dev, name="workspace"):
    """A caller's workspace (uint8, on dev, at least nbytes) or a new one."""
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(ws, name, torch.uint8, 1, dev)
    if ws.numel() < nbytes:
        raise ValueError(f"{name} holds {ws.numel()} bytes, {nbytes} needed")
    return ws


def _call(status, what):
    if status != 0:
        raise DmaError(status, what)


def dt(V, W, A, bias=None, out=None, out_pos=None):
    """dt = exp(A * softplus(dt_proj(V))) -> float32 [B, Hkv, S] (or written into `out`)."""
    _check(V, "V", ndim=4)
    dev = V.device
    _check(W, "W", V.dtype, 2, dev)
    _check(A, "A", torch.float32, 1, dev)
    if bias is not None:
        _check(bias, "bias", V.dtype, 1, dev)
    B, S, Hkv, d = V.shape
    _shape(W, "W", (Hkv, Hkv * d))
    _shape(A, "A", (Hkv,))
    if bias is not None:
        _shape(bias, "bias", (Hkv,))
    if out_pos is not None:
        _check(out_pos, "out_pos", torch.int32, 1, dev)
        _shape(out_pos, "out_pos", (B,))
    if out is not None:
        _check(out, "out", torch.float32, 3, dev)
        if out.shape[0] != B or out.shape[1] != Hkv or out.shape[2] < S:
            raise ValueError(f"out must be [B={B}, Hkv={Hkv}, >= S={S}], got {tuple(out.shape)}")
    else:
        out = torch.empty((B, Hkv, S), dtype=torch.float32, device=dev)
    ld = out.shape[2]
    _call(lib().dma_dt(_ptr(V), _ptr(W), _ptr(bias), _ptr(A), _dtype_code(V), B, S, Hkv, d,
                       _ptr(out), ld, _ptr(out_pos), _stream(V)), "dma_dt")
    return out


def _select_args(dt_, seqlens, tau, tie):
    B, Hkv, S = dt_.shape
    dev = dt_.device
    if seqlens is not None:
        _check(seqlens, "seqlens", torch.int32, 1, dev)
        _shape(seqlens, "seqlens", (B,))
    for name, t, dtp in (("tau", tau, torch.float32), ("tie", tie, torch.int32)):
        if t is not None:
            _check(t, name, dtp, 3, dev)
            _shape(t, name, (B, Hkv, S))
    if tau is None:
        tau = torch.empty_like(dt_)
    if tie is None:
        tie = torch.empty((B, Hkv, S), dtype=torch.int32, device=dev)
    return tau, tie


def select(dt_, w, seqlens=None, tau=None, tie=None):
    """Per-row threshold pairs (tau float32, tie int32), each [B, Hkv, S]."""
    _check(dt_, "dt", torch.float32, 3)
    B, Hkv, S = dt_.shape
    tau, tie = _select_args(dt_, seqlens, tau, tie)
    _call(lib().dma_select(_ptr(dt_), _ptr(seqlens), B, Hkv, S, int(w), _ptr(tau), _ptr(tie),
                           _stream(dt_)), "dma_select")
    return tau, tie


def attn_fwd(Q, K, V, dt_, tau, tie, w, seqlens=None, out=None):
    """Masked attention output O [B, S, Hq, d] in the dtype of Q."""
    _check(Q, "Q", ndim=4)
    dev = Q.device
    _check(K, "K", Q.dtype, 4, dev)
    _check(V, "V", Q.dtype, 4, dev)
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    if tuple(K.shape) != (B, S, Hkv, d) or tuple(V.shape) != tuple(K.shape):
        raise ValueError("K/V must be [B, S, Hkv, d] matching Q")
    for name, t, dtp in (("dt", dt_, torch.float32), ("tau", tau, torch.float32), ("tie", tie, torch.int32)):
        _check(t, name, dtp, 3, dev)
        if tuple(t.shape) != (B, Hkv, S):
            raise ValueError(f"{name} must be [B, Hkv, S]")
    if seqlens is not None:
        _check(seqlens, "seqlens", torch.int32, 1, dev)
        _shape(seqlens, "seqlens", (B,))
    if out is None:
        out = torch.empty_like(Q)
    _check(out, "out", Q.dtype, 4, dev)
    _shape(out, "out", Q.shape)
    _call(lib().dma_attn_fwd(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), _ptr(dt_), _ptr(tau), _ptr(tie),
                             _ptr(seqlens), B, S, Hq, Hkv, d, int(w), _ptr(out), _stream(Q)),
          "dma_attn_fwd")
    return out


OP_DT, OP_SELECT, OP_ATTN_FWD, OP_DECODE, OP_DECODE_STEP, OP_ATTN_BWD, OP_DT_BWD = range(7)


def workspace_bytes(op, B, S, Hq, Hkv, d, w):
    """Device workspace of operation `op` (OP_*) in bytes; 0 when it takes none.
    Raises ValueError for an unknown op or sizes the operation rejects."""
    n = int(lib().dma_workspace_bytes(int(op), B, S, Hq, Hkv, d, int(w)))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError(f"dma_workspace_bytes: op {op} rejects sizes B={B} S={S} Hq={Hq} Hkv={Hkv} d={d} w={w}")
    return n


def decode_workspace_bytes(B, Lmax, Hq, Hkv, d, w):
    return int(lib().dma_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, w))


def decode(q, Kc, Vc, dt_cache, cache_lens, w, kept=False, out=None, workspace=None):
    """One decode step: out [B, Hq, d]; with kept=True also kept_idx [B, Hkv, w] int32."""
    _check(q, "q", ndim=3)
    dev = q.device
    _check(Kc, "Kc", q.dtype, 4, dev)
    _check(Vc, "Vc", q.dtype, 4, dev)
    _check(dt_cache, "dt_cache", torch.float32, 3, dev)
    _check(cache_lens, "cache_lens", torch.int32, 1, dev)
    B, Hq, d = q.shape
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    _shape(Kc, "Kc", (B, Lmax, Hkv, d))
    _shape(Vc, "Vc", Kc.shape)
    _shape(dt_cache, "dt_cache", (B, Hkv, Lmax))
    _shape(cache_lens, "cache_lens", (B,))
    if out is not None:
        _check(out, "out", q.dtype, 3, dev)
        _shape(out, "out", q.shape)
    nbytes = decode_workspace_bytes(B, Lmax, Hq, Hkv, d, w)
    workspace = _workspace(workspace, nbytes, dev)
    if out is None:
        out = torch.empty_like(q)
    kept_idx = torch.empty((B, Hkv, int(w)), dtype=torch.int32, device=dev) if kept else None
    _call(lib().dma_decode(_ptr(q), _ptr(Kc), _ptr(Vc), _dtype_code(q), _ptr(dt_cache), _ptr(cache_lens),
                           B, Lmax, Hq, Hkv, d, int(w), _ptr(out), _ptr(kept_idx), _ptr(workspace),
                           workspace.numel(), _stream(q)), "dma_decode")
    return (out, kept_idx) if kept else out


DECODE_NOALLOC_MAX_WORKSPACE = 16 << 20


def decode_noalloc(q, Kc, Vc, dt_cache, cache_lens, w, kept=False, out=None):
    """decode() through dma_decode_noalloc: no workspace is allocated (the library's static device
    array serves instead; sizes needing more than 16 MiB of workspace are rejected).  Outputs are
    allocated here unless given; calls that overlap in time on one device race."""
    _check(q, "q", ndim=3)
    dev = q.device
    _check(Kc, "Kc", q.dtype, 4, dev)
    _check(Vc, "Vc", q.dtype, 4, dev)
    _check(dt_cache, "dt_cache", torch.float32, 3, dev)
    _check(cache_lens, "cache_lens", torch.int32, 1, dev)
    B, Hq, d = q.shape
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    _shape(Kc, "Kc", (B, Lmax, Hkv, d))
    _shape(Vc, "Vc", Kc.shape)
    _shape(dt_cache, "dt_cache", (B, Hkv, Lmax))
    _shape(cache_lens, "cache_lens", (B,))
    if out is not None:
        _check(out, "out", q.dtype, 3, dev)
        _shape(out, "out", q.shape)
    else:
        out = torch.empty_like(q)
    kept_idx = torch.empty((B, Hkv, int(w)), dtype=torch.int32, device=dev) if kept else None
    _call(lib().dma_decode_noalloc(_ptr(q), _ptr(Kc), _ptr(Vc), _dtype_code(q), _ptr(dt_cache), _ptr(cache_lens),
                                   B, Lmax, Hq, Hkv, d, int(w), _ptr(out), _ptr(kept_idx), _stream(q)),
          "dma_decode_noalloc")
    return (out, kept_idx) if kept else out


def prefill(Q, K, V, W, A, w, bias=None, seqlens=None):
    """The whole prefill path: dt from V, per-row thresholds, masked attention."""
    d_ = dt(V, W, A, bias)
    tau, tie = select(d_, w, seqlens)
    O = attn_fwd(Q, K, V, d_, tau, tie, w, seqlens)
    return O, d_, tau, tie


class DecodeState:
    """Kept keys of every (batch, kv head), carried from one decode step to the next.

    Built from a cache by decode_state_init(); advanced one token per batch by
    decode_step().  Holds the device buffers and the sizes they were made for."""

    def __init__(self, B, Hkv, d, w, device):
        self.B, self.Hkv, self.d, self.w = B, Hkv, d, int(w)
        n = int(lib().dma_decode_state_bytes(B, Hkv, d, self.w))
        if n == 0:
            raise ValueError("invalid decode state sizes")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)

    def kept(self):
        """(kept positions [B, Hkv, w] int32 in slot order, -1 padded; lengths [B, Hkv] int32)."""
        dev = self.buf.device
        kept_idx = torch.empty((self.B, self.Hkv, self.w), dtype=torch.int32, device=dev)
        lens = torch.empty((self.B, self.Hkv), dtype=torch.int32, device=dev)
        _call(lib().dma_decode_state_kept(_ptr(self.buf), self.buf.numel(), self.B, self.Hkv, self.d, self.w,
                                          _ptr(kept_idx), _ptr(lens), _stream(self.buf)), "dma_decode_state_kept")
        return kept_idx, lens


def decode_step_workspace_bytes(B, Hq, Hkv, d, w):
    return int(lib().dma_decode_step_workspace_bytes(B, Hq, Hkv, d, w))


def decode_state_init(Kc, Vc, dt_cache, cache_lens, w, state=None, workspace=None):
    """The DecodeState of a cache of cache_lens[b] positions (bf16 K/V)."""
    _check(Kc, "Kc", torch.bfloat16, 4)
    dev = Kc.device
    _check(Vc, "Vc", torch.bfloat16, 4, dev)
    _check(dt_cache, "dt_cache", torch.float32, 3, dev)
    _check(cache_lens, "cache_lens", torch.int32, 1, dev)
    B, Lmax, Hkv, d = Kc.shape
    _shape(Vc, "Vc", Kc.shape)
    _shape(dt_cache, "dt_cache", (B, Hkv, Lmax))
    _shape(cache_lens, "cache_lens", (B,))
    if state is not None and (state.B, state.Hkv, state.d, state.w) != (B, Hkv, d, int(w)):
        raise ValueError("the decode state was made for other sizes")
    nbytes = decode_step_workspace_bytes(B, Hkv, Hkv, d, w)
    workspace = _workspace(workspace, nbytes, dev)
    if state is None:
        state = DecodeState(B, Hkv, d, w, dev)
    _call(lib().dma_decode_state_init(_ptr(Kc), _ptr(Vc), BF16, _ptr(dt_cache), _ptr(cache_lens), B, Lmax, Hkv, d,
                                      int(w), _ptr(state.buf), state.buf.numel(), _ptr(workspace),
                                      workspace.numel(), _stream(Kc)), "dma_decode_state_init")
    return state


def decode_step(q, k_new, v_new, dt_new, state, out=None, workspace=None):
    """Append one token per batch (rows k_new/v_new [B, Hkv, d], dt_new [B, Hkv]) and decode q [B, Hq, d]."""
    _check(q, "q", torch.bfloat16, 3)
    dev = q.device
    _check(k_new, "k_new", torch.bfloat16, 3, dev)
    _check(v_new, "v_new", torch.bfloat16, 3, dev)
    _check(dt_new, "dt_new", torch.float32, 2, dev)
    B, Hq, d = q.shape
    Hkv = state.Hkv
    if (B, d) != (state.B, state.d):
        raise ValueError("q does not match the decode state")
    _shape(k_new, "k_new", (B, Hkv, d))
    _shape(v_new, "v_new", (B, Hkv, d))
    _shape(dt_new, "dt_new", (B, Hkv))
    if state.buf.device != dev:
        raise ValueError(f"the decode state is on {state.buf.device}, expected {dev}")
    if out is not None:
        _check(out, "out", q.dtype, 3, dev)
        _shape(out, "out", q.shape)
    nbytes = decode_step_workspace_bytes(B, Hq, Hkv, d, state.w)
    workspace = _workspace(workspace, nbytes, dev)
    if out is None:
        out = torch.empty_like(q)
    _call(lib().dma_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), BF16, _ptr(dt_new), B, Hq, Hkv, d, state.w,
                                _ptr(state.buf), state.buf.numel(), _ptr(out), _ptr(workspace), workspace.numel(),
                                _stream(q)), "dma_decode_step")
    return out


def _qk_args(Q, K, q_norm_w, k_norm_w, positions, Q_out, K_out):
    _check(Q, "Q", ndim=4)
    dev = Q.device
    _check(K, "K", Q.dtype, 4, dev)
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    if tuple(K.shape) != (B, S, Hkv, d):
        raise ValueError("K must be [B, S, Hkv, d] matching Q")
    _check(q_norm_w, "q_norm_w", Q.dtype, 1, dev)
    _check(k_norm_w, "k_norm_w", Q.dtype, 1, dev)
    if q_norm_w.shape[0] != d or k_norm_w.shape[0] != d:
        raise ValueError("q_norm_w / k_norm_w must have head_dim elements")
    if positions is not None:
        _check(positions, "positions", torch.int32, 2, dev)
        if tuple(positions.shape) != (B, S):
            raise ValueError("positions must be [B, S]")
    Q_out = torch.empty_like(Q) if Q_out is None else Q_out
    K_out = torch.empty_like(K) if K_out is None else K_out
    _check(Q_out, "Q_out", Q.dtype, 4, dev)
    _check(K_out, "K_out", Q.dtype, 4, dev)
    if Q_out.shape != Q.shape or K_out.shape != K.shape:
        raise ValueError("Q_out / K_out must have the shapes of Q / K")
    return B, S, Hq, Hkv, d, Q_out, K_out


def qk_norm_rope(Q, K, q_norm_w, k_norm_w, eps=1e-6, rope_theta=10000.0, positions=None, Q_out=None, K_out=None):
    """RMSNorm over head_dim (weights q_norm_w / k_norm_w) then rotary embedding of Q [B,S,Hq,d] and
    K [B,S,Hkv,d] at positions [B,S] int32 (None: position s).  Q_out=Q, K_out=K runs in place."""
    B, S, Hq, Hkv, d, Q_out, K_out = _qk_args(Q, K, q_norm_w, k_norm_w, positions, Q_out, K_out)
    _call(lib().dma_qk_norm_rope(_ptr(Q), _ptr(K), _dtype_code(Q), _ptr(q_norm_w), _ptr(k_norm_w), float(eps),
                                 float(rope_theta), _ptr(positions), B, S, Hq, Hkv, d, _ptr(Q_out), _ptr(K_out),
                                 _stream(Q)), "dma_qk_norm_rope")
    return Q_out, K_out


def prologue(Q, K, V, q_norm_w, k_norm_w, W, A, bias=None, eps=1e-6, rope_theta=10000.0, positions=None,
             Q_out=None, K_out=None, dt_out=None):
    """qk_norm_rope on Q and K plus dt from V, in one call -> (Q', K', dt [B, Hkv, S] float32)."""
    B, S, Hq, Hkv, d, Q_out, K_out = _qk_args(Q, K, q_norm_w, k_norm_w, positions, Q_out, K_out)
    dev = Q.device
    _check(V, "V", Q.dtype, 4, dev)
    if tuple(V.shape) != tuple(K.shape):
        raise ValueError("V must be [B, S, Hkv, d] matching K")
    _check(W, "W", Q.dtype, 2, dev)
    _check(A, "A", torch.float32, 1, dev)
    _shape(W, "W", (Hkv, Hkv * d))
    _shape(A, "A", (Hkv,))
    if bias is not None:
        _check(bias, "bias", Q.dtype, 1, dev)
        _shape(bias, "bias", (Hkv,))
    if dt_out is None:
        dt_out = torch.empty((B, Hkv, S), dtype=torch.float32, device=dev)
    _check(dt_out, "dt_out", torch.float32, 3, dev)
    if tuple(dt_out.shape) != (B, Hkv, S):
        raise ValueError("dt_out must be [B, Hkv, S]")
    _call(lib().dma_prologue(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), _ptr(q_norm_w), _ptr(k_norm_w), float(eps),
                             float(rope_theta), _ptr(positions), _ptr(W), _ptr(bias), _ptr(A), B, S, Hq, Hkv, d,
                             _ptr(Q_out), _ptr(K_out), _ptr(dt_out), _stream(Q)), "dma_prologue")
    return Q_out, K_out, dt_out


def attn_bwd_workspace_bytes(B, S, Hq, Hkv, d, w):
    return int(lib().dma_attn_bwd_workspace_bytes(B, S, Hq, Hkv, d, w))


def attn_bwd(Q, K, V, dt_, tau, tie, w, dO, seqlens=None, workspace=None, out=None):
    """Gradients of attn_fwd for the upstream gradient dO: (dQ, dK, dV) in the dtype of Q and
    ddt [B, Hkv, S] float32 (bf16 only)."""
    _check(Q, "Q", torch.bfloat16, 4)
    dev = Q.device
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    for name, t in (("K", K), ("V", V)):
        _check(t, name, Q.dtype, 4, dev)
        if tuple(t.shape) != (B, S, Hkv, d):
            raise ValueError(f"{name} must be [B, S, Hkv, d] matching Q")
    _check(dO, "dO", Q.dtype, 4, dev)
    if dO.shape != Q.shape:
        raise ValueError("dO must have the shape of Q")
    for name, t, dtp in (("dt", dt_, torch.float32), ("tau", tau, torch.float32), ("tie", tie, torch.int32)):
        _check(t, name, dtp, 3, dev)
        if tuple(t.shape) != (B, Hkv, S):
            raise ValueError(f"{name} must be [B, Hkv, S]")
    if seqlens is not None:
        _check(seqlens, "seqlens", torch.int32, 1, dev)
        _shape(seqlens, "seqlens", (B,))
    if out is not None:
        dQ, dK, dV, ddt = out
        for name, t, ref in (("dQ", dQ, Q), ("dK", dK, K), ("dV", dV, V)):
            _check(t, name, Q.dtype, 4, dev)
            _shape(t, name, ref.shape)
        _check(ddt, "ddt", torch.float32, 3, dev)
        _shape(ddt, "ddt", (B, Hkv, S))
    nbytes = attn_bwd_workspace_bytes(B, S, Hq, Hkv, d, w)
    workspace = _workspace(workspace, nbytes, dev)
    if out is None:
        out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V),
               torch.empty((B, Hkv, S), dtype=torch.float32, device=dev))
    dQ, dK, dV, ddt = out
    _call(lib().dma_attn_bwd(_ptr(Q), _ptr(K), _ptr(V), BF16, _ptr(dt_), _ptr(tau), _ptr(tie), _ptr(seqlens),
                             _ptr(dO), B, S, Hq, Hkv, d, int(w), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ddt),
                             _ptr(workspace), workspace.numel(), _stream(Q)), "dma_attn_bwd")
    return dQ, dK, dV, ddt


def dt_bwd_workspace_bytes(B, S, Hkv, d):
    return int(lib().dma_dt_bwd_workspace_bytes(B, S, Hkv, d))


def dt_bwd(V, W, A, ddt, bias=None, dV=None, workspace=None):
    """Gradients of dt() for the upstream gradient ddt [B, Hkv, S] float32: (dW, dbias, dA) float32.
    If dV [B, S, Hkv, d] (dtype of V) is given, the dt path's part of the value gradient is added to it."""
    _check(V, "V", ndim=4)
    dev = V.device
    _check(W, "W", V.dtype, 2, dev)
    _check(A, "A", torch.float32, 1, dev)
    _check(ddt, "ddt", torch.float32, 3, dev)
    B, S, Hkv, d = V.shape
    if tuple(ddt.shape) != (B, Hkv, S):
        raise ValueError("ddt must be [B, Hkv, S]")
    _shape(W, "W", (Hkv, Hkv * d))
    _shape(A, "A", (Hkv,))
    if bias is not None:
        _check(bias, "bias", V.dtype, 1, dev)
        _shape(bias, "bias", (Hkv,))
    if dV is not None:
        _check(dV, "dV", V.dtype, 4, dev)
        if dV.shape != V.shape:
            raise ValueError("dV must have the shape of V")
    nbytes = dt_bwd_workspace_bytes(B, S, Hkv, d)
    workspace = _workspace(workspace, nbytes, dev)
    dW = torch.empty((Hkv, Hkv * d), dtype=torch.float32, device=dev)
    dbias = torch.empty(Hkv, dtype=torch.float32, device=dev)
    dA = torch.empty(Hkv, dtype=torch.float32, device=dev)
    _call(lib().dma_dt_bwd(_ptr(V), _ptr(W), _ptr(bias), _ptr(A), _dtype_code(V), _ptr(ddt), B, S, Hkv, d,
                           _ptr(dV), _ptr(dW), _ptr(dbias), _ptr(dA), _ptr(workspace), workspace.numel(),
                           _stream(V)), "dma_dt_bwd")
    return dW, dbias, dA


def prefill_bwd(Q, K, V, W, A, w, dO, bias=None, seqlens=None, fwd=None):
    """Every gradient of prefill() for the upstream gradient dO: dQ, dK, dV (attention and dt path),
    dW, dbias, dA and ddt.  fwd = (dt, tau, tie) of the forward, recomputed when None."""
    if fwd is None:
        d_ = dt(V, W, A, bias)
        tau, tie = select(d_, w, seqlens)
    else:
        d_, tau, tie = fwd
    dQ, dK, dV, ddt = attn_bwd(Q, K, V, d_, tau, tie, w, dO, seqlens)
    dW, dbias, dA = dt_bwd(V, W, A, ddt, bias, dV=dV)
    return {"dQ": dQ, "dK": dK, "dV": dV, "dW": dW, "dbias": dbias, "dA": dA, "ddt": ddt}


def select_window(dt_, w, win, seqlens=None, tau=None, tie=None):
    """Per-row threshold pairs under a sliding window of win positions: (tau, tie), each [B, Hkv, S]."""
    _check(dt_, "dt", torch.float32, 3)
    B, Hkv, S = dt_.shape
    tau, tie = _select_args(dt_, seqlens, tau, tie)
    _call(lib().dma_select_window(_ptr(dt_), _ptr(seqlens), B, Hkv, S, int(w), int(win), _ptr(tau), _ptr(tie),
                                  _stream(dt_)), "dma_select_window")
    return tau, tie


def attn_window_fwd(Q, K, V, dt_, tau, tie, w, win, seqlens=None, out=None):
    """Masked attention under a sliding window of win positions: O [B, S, Hq, d] (bf16)."""
    _check(Q, "Q", torch.bfloat16, 4)
    dev = Q.device
    B, S, Hq, d = Q.shape
    Hkv = K.shape[2]
    for name, t in (("K", K), ("V", V)):
        _check(t, name, Q.dtype, 4, dev)
        if tuple(t.shape) != (B, S, Hkv, d):
            raise ValueError(f"{name} must be [B, S, Hkv, d] matching Q")
    for name, t, dtp in (("dt", dt_, torch.float32), ("tau", tau, torch.float32), ("tie", tie, torch.int32)):
        _check(t, name, dtp, 3, dev)
        if tuple(t.shape) != (B, Hkv, S):
            raise ValueError(f"{name} must be [B, Hkv, S]")
    if seqlens is not None:
        _check(seqlens, "seqlens", torch.int32, 1, dev)
        _shape(seqlens, "seqlens", (B,))
    if out is None:
        out = torch.empty_like(Q)
    _check(out, "out", Q.dtype, 4, dev)
    _shape(out, "out", Q.shape)
    _call(lib().dma_attn_window_fwd(_ptr(Q), _ptr(K), _ptr(V), BF16, _ptr(dt_), _ptr(tau), _ptr(tie), _ptr(seqlens),
                                    B, S, Hq, Hkv, d, int(w), int(win), _ptr(out), _stream(Q)), "dma_attn_window_fwd")
    return out


def cdmoe_logits(h, router, out=None):
    """Router logits [T, 2*nk] float32 of hidden states h [T, H] (bf16) for router [2*nk, H]."""
    _check(h, "h", torch.bfloat16, 2)
    _check(router, "router", torch.bfloat16, 2, h.device)
    T, H = h.shape
    n2 = router.shape[0]
    if router.shape[1] != H or n2 % 2:
        raise ValueError("router must be [2*nk, H]")
    if out is None:
        out = torch.empty((T, n2), dtype=torch.float32, device=h.device)
    _check(out, "out", torch.float32, 2, h.device)
    _shape(out, "out", (T, n2))
    _call(lib().dma_cdmoe_logits(_ptr(h), _ptr(router), BF16, T, H, n2 // 2, _ptr(out), _stream(h)),
          "dma_cdmoe_logits")
    return out


def cdmoe_route(logits, k, idx=None, weights=None):
    """Product-key routing: (expert indices [T, k] int32 best first, weights [T, k] float32)."""
    _check(logits, "logits", torch.float32, 2)
    T, n2 = logits.shape
    if n2 % 2:
        raise ValueError("logits must be [T, 2*nk]")
    for name, t, dtp in (("idx", idx, torch.int32), ("weights", weights, torch.float32)):
        if t is not None:
            _check(t, name, dtp, 2, logits.device)
            _shape(t, name, (T, int(k)))
    if idx is None:
        idx = torch.empty((T, int(k)), dtype=torch.int32, device=logits.device)
    if weights is None:
        weights = torch.empty((T, int(k)), dtype=torch.float32, device=logits.device)
    _call(lib().dma_cdmoe_route(_ptr(logits), T, n2 // 2, int(k), _ptr(idx), _ptr(weights), _stream(logits)),
          "dma_cdmoe_route")
    return idx, weights


def cdmoe_experts(h, down, up, idx, weights, out=None):
    """sum_e weights * silu(down[idx] . h) * up[idx] per token: [T, H] bf16."""
    _check(h, "h", torch.bfloat16, 2)
    dev = h.device
    _check(down, "down", torch.bfloat16, 2, dev)
    _check(up, "up", torch.bfloat16, 2, dev)
    _check(idx, "idx", torch.int32, 2, dev)
    _check(weights, "weights", torch.float32, 2, dev)
    T, H = h.shape
    E = down.shape[0]
    nk = int(round(E ** 0.5))
    if nk * nk != E or tuple(up.shape) != (E, H) or down.shape[1] != H:
        raise ValueError("down/up must be [nk*nk, H]")
    if idx.shape[0] != T or weights.shape != idx.shape:
        raise ValueError("idx/weights must be [T, k]")
    if out is None:
        out = torch.empty_like(h)
    _check(out, "out", torch.bfloat16, 2, dev)
    _shape(out, "out", h.shape)
    _call(lib().dma_cdmoe_experts(_ptr(h), _ptr(down), _ptr(up), BF16, _ptr(idx), _ptr(weights), T, H, nk,
                                  idx.shape[1], _ptr(out), _stream(h)), "dma_cdmoe_experts")
    return out

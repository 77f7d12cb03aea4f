"""The Python binding rejects mismatched shapes before it calls the library.

Runs without a GPU: the binding's device check is relaxed to accept CPU
tensors, the stream lookup returns NULL and the library is replaced by a
recorder, so each case shows whether a call would have reached libdma.so.
Every mismatch below would otherwise hand the kernels a buffer smaller than
the sizes they are told, i.e. an out-of-bounds read or write on the device.
"""
import pytest
import torch

import doge_dynamic_mask_amd as dma


class _Recorder:
    """Stands in for the ctypes library: records calls, returns DMA_OK and
    plausible workspace sizes."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        if not name.startswith("dma_"):
            raise AttributeError(name)

        def f(*args):
            if name.endswith("_bytes"):
                return 4096
            self.calls.append(name)
            return 0
        return f


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder()
    real_check = dma._check

    def check(t, name, dtype=None, ndim=None, device=None):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if ndim is not None and t.dim() != ndim:
            raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    assert real_check is not None
    monkeypatch.setattr(dma, "_check", check)
    monkeypatch.setattr(dma, "lib", lambda: r)
    monkeypatch.setattr(dma, "_stream", lambda t: None)
    return r


BF, F32, I32 = torch.bfloat16, torch.float32, torch.int32


def z(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


def expect_reject(rec, fn, *args, **kw):
    n = len(rec.calls)
    with pytest.raises(ValueError):
        fn(*args, **kw)
    assert len(rec.calls) == n, "the library was called despite the mismatch"


def test_dt_shapes(rec):
    B, S, Hkv, d = 2, 16, 4, 64
    V, W, A = z(B, S, Hkv, d), z(Hkv, Hkv * d), z(Hkv, dtype=F32)
    dma.dt(V, W, A)
    dma.dt(V, W, A, bias=z(Hkv), out=z(B, Hkv, 64, dtype=F32), out_pos=z(B, dtype=I32))
    assert rec.calls == ["dma_dt", "dma_dt"]
    expect_reject(rec, dma.dt, V, z(Hkv, d), A)                      # W not [Hkv, Hkv*d]
    expect_reject(rec, dma.dt, V, W, z(Hkv + 1, dtype=F32))          # A too long
    expect_reject(rec, dma.dt, V, W, A, bias=z(Hkv - 1))
    expect_reject(rec, dma.dt, V, W, A, out=z(B, Hkv, S - 1, dtype=F32))
    expect_reject(rec, dma.dt, V, W, A, out=z(B - 1, Hkv, S, dtype=F32))
    expect_reject(rec, dma.dt, V, W, A, out=z(B, Hkv + 1, S, dtype=F32))
    expect_reject(rec, dma.dt, V, W, A, out=z(B, Hkv, S, dtype=F32), out_pos=z(B + 1, dtype=I32))


def test_select_shapes(rec):
    B, Hkv, S = 2, 4, 32
    dt_ = z(B, Hkv, S, dtype=F32)
    dma.select(dt_, 8)
    dma.select(dt_, 8, z(B, dtype=I32), tau=z(B, Hkv, S, dtype=F32), tie=z(B, Hkv, S, dtype=I32))
    assert rec.calls == ["dma_select"] * 2
    expect_reject(rec, dma.select, dt_, 8, z(B + 1, dtype=I32))
    expect_reject(rec, dma.select, dt_, 8, tau=z(B, Hkv, S - 1, dtype=F32))
    expect_reject(rec, dma.select, dt_, 8, tie=z(B, Hkv + 1, S, dtype=I32))
    expect_reject(rec, dma.select_window, dt_, 8, 16, z(B - 1, dtype=I32))


def test_attn_fwd_shapes(rec):
    B, S, Hq, Hkv, d = 2, 32, 8, 4, 64
    Q, K, V = z(B, S, Hq, d), z(B, S, Hkv, d), z(B, S, Hkv, d)
    dt_, tau, tie = z(B, Hkv, S, dtype=F32), z(B, Hkv, S, dtype=F32), z(B, Hkv, S, dtype=I32)
    dma.attn_fwd(Q, K, V, dt_, tau, tie, 8)
    dma.attn_fwd(Q, K, V, dt_, tau, tie, 8, z(B, dtype=I32), out=z(B, S, Hq, d))
    assert rec.calls == ["dma_attn_fwd"] * 2
    expect_reject(rec, dma.attn_fwd, Q, K, z(B, S, Hkv, 2 * d), dt_, tau, tie, 8)
    expect_reject(rec, dma.attn_fwd, Q, K, V, z(B, Hkv, S + 1, dtype=F32), tau, tie, 8)
    expect_reject(rec, dma.attn_fwd, Q, K, V, dt_, tau, tie, 8, z(B + 1, dtype=I32))
    expect_reject(rec, dma.attn_fwd, Q, K, V, dt_, tau, tie, 8, out=z(B, S, Hq - 1, d))
    expect_reject(rec, dma.attn_window_fwd, Q, K, V, dt_, tau, tie, 8, 16, out=z(B, S - 1, Hq, d))
    expect_reject(rec, dma.attn_window_fwd, Q, K, V, dt_, tau, tie, 8, 16, z(3, dtype=I32))


def test_decode_shapes(rec):
    B, Lmax, Hq, Hkv, d, w = 3, 64, 8, 2, 128, 16
    q, Kc, Vc = z(B, Hq, d), z(B, Lmax, Hkv, d), z(B, Lmax, Hkv, d)
    dtc, lens = z(B, Hkv, Lmax, dtype=F32), z(B, dtype=I32)
    dma.decode(q, Kc, Vc, dtc, lens, w)
    dma.decode(q, Kc, Vc, dtc, lens, w, kept=True, out=z(B, Hq, d), workspace=z(4096, dtype=torch.uint8))
    assert rec.calls == ["dma_decode"] * 2
    expect_reject(rec, dma.decode, q, z(B - 1, Lmax, Hkv, d), z(B - 1, Lmax, Hkv, d), dtc, lens, w)
    expect_reject(rec, dma.decode, q, z(B, Lmax, Hkv, d // 2), z(B, Lmax, Hkv, d // 2), dtc, lens, w)
    expect_reject(rec, dma.decode, q, Kc, z(B, Lmax - 1, Hkv, d), dtc, lens, w)
    expect_reject(rec, dma.decode, q, Kc, Vc, z(B, Hkv, Lmax - 1, dtype=F32), lens, w)
    expect_reject(rec, dma.decode, q, Kc, Vc, dtc, z(B + 1, dtype=I32), w)
    expect_reject(rec, dma.decode, q, Kc, Vc, dtc, lens, w, out=z(B, Hq, d - 1))
    expect_reject(rec, dma.decode, q, Kc, Vc, dtc, lens, w, workspace=z(100, dtype=torch.uint8))


def test_decode_state_shapes(rec, monkeypatch):
    B, Lmax, Hq, Hkv, d, w = 2, 64, 8, 2, 128, 16
    Kc, Vc = z(B, Lmax, Hkv, d), z(B, Lmax, Hkv, d)
    dtc, lens = z(B, Hkv, Lmax, dtype=F32), z(B, dtype=I32)
    st = dma.decode_state_init(Kc, Vc, dtc, lens, w)
    assert rec.calls == ["dma_decode_state_init"]
    expect_reject(rec, dma.decode_state_init, Kc, z(B, Lmax, Hkv, d // 2), dtc, lens, w)
    expect_reject(rec, dma.decode_state_init, Kc, Vc, z(B, Hkv, Lmax + 1, dtype=F32), lens, w)
    expect_reject(rec, dma.decode_state_init, Kc, Vc, dtc, z(B - 1, dtype=I32), w)
    expect_reject(rec, dma.decode_state_init, Kc, Vc, dtc, lens, w + 1, state=st)
    q, kn, vn, dn = z(B, Hq, d), z(B, Hkv, d), z(B, Hkv, d), z(B, Hkv, dtype=F32)
    dma.decode_step(q, kn, vn, dn, st)
    assert rec.calls[-1] == "dma_decode_step"
    expect_reject(rec, dma.decode_step, z(B + 1, Hq, d), kn, vn, dn, st)
    expect_reject(rec, dma.decode_step, q, z(B, Hkv + 1, d), vn, dn, st)
    expect_reject(rec, dma.decode_step, q, kn, z(B, Hkv, d // 2), dn, st)
    expect_reject(rec, dma.decode_step, q, kn, vn, z(B, Hkv - 1, dtype=F32), st)
    expect_reject(rec, dma.decode_step, q, kn, vn, dn, st, out=z(B, Hq - 1, d))


def test_backward_shapes(rec):
    B, S, Hq, Hkv, d = 2, 32, 8, 4, 64
    Q, K, V, dO = z(B, S, Hq, d), z(B, S, Hkv, d), z(B, S, Hkv, d), z(B, S, Hq, d)
    dt_, tau, tie = z(B, Hkv, S, dtype=F32), z(B, Hkv, S, dtype=F32), z(B, Hkv, S, dtype=I32)
    dma.attn_bwd(Q, K, V, dt_, tau, tie, 8, dO)
    assert rec.calls == ["dma_attn_bwd"]
    expect_reject(rec, dma.attn_bwd, Q, K, V, dt_, tau, tie, 8, dO, z(B + 1, dtype=I32))
    bad_out = (z(B, S, Hq, d), z(B, S, Hkv, d), z(B, S, Hkv, d), z(B, Hkv, S - 1, dtype=F32))
    expect_reject(rec, dma.attn_bwd, Q, K, V, dt_, tau, tie, 8, dO, out=bad_out)
    bad_out = (z(B, S, Hq, d), z(B, S - 1, Hkv, d), z(B, S, Hkv, d), z(B, Hkv, S, dtype=F32))
    expect_reject(rec, dma.attn_bwd, Q, K, V, dt_, tau, tie, 8, dO, out=bad_out)
    W, A, ddt = z(Hkv, Hkv * d), z(Hkv, dtype=F32), z(B, Hkv, S, dtype=F32)
    dma.dt_bwd(V, W, A, ddt, dV=z(B, S, Hkv, d))
    assert rec.calls[-1] == "dma_dt_bwd"
    expect_reject(rec, dma.dt_bwd, V, z(Hkv, d), A, ddt)
    expect_reject(rec, dma.dt_bwd, V, W, z(Hkv + 2, dtype=F32), ddt)
    expect_reject(rec, dma.dt_bwd, V, W, A, ddt, bias=z(Hkv + 1))


def test_prologue_and_cdmoe_shapes(rec):
    B, S, Hq, Hkv, d = 2, 16, 8, 4, 64
    Q, K, V = z(B, S, Hq, d), z(B, S, Hkv, d), z(B, S, Hkv, d)
    wq, wk, W, A = z(d), z(d), z(Hkv, Hkv * d), z(Hkv, dtype=F32)
    dma.prologue(Q, K, V, wq, wk, W, A)
    assert rec.calls == ["dma_prologue"]
    expect_reject(rec, dma.prologue, Q, K, V, wq, wk, z(Hkv, d), A)
    expect_reject(rec, dma.prologue, Q, K, V, wq, wk, W, z(Hkv - 1, dtype=F32))
    T, H, nk, k = 8, 512, 16, 4
    h, router = z(T, H), z(2 * nk, H)
    dma.cdmoe_logits(h, router)
    expect_reject(rec, dma.cdmoe_logits, h, router, out=z(T, 2 * nk - 2, dtype=F32))
    lg = z(T, 2 * nk, dtype=F32)
    dma.cdmoe_route(lg, k)
    expect_reject(rec, dma.cdmoe_route, lg, k, idx=z(T, k + 1, dtype=I32))
    expect_reject(rec, dma.cdmoe_route, z(T, 2 * nk + 1, dtype=F32), k)
    down, up, idx, wts = z(nk * nk, H), z(nk * nk, H), z(T, k, dtype=I32), z(T, k, dtype=F32)
    dma.cdmoe_experts(h, down, up, idx, wts)
    expect_reject(rec, dma.cdmoe_experts, h, down, up, idx, wts, out=z(T, H - 1))
    expect_reject(rec, dma.cdmoe_experts, h, down, up, idx, z(T, k + 1, dtype=F32))

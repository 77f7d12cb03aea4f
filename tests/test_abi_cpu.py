"""The C ABI library without a GPU: it loads, exports every function that
include/dma.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dma.h")
LIB = os.path.join(ROOT, "doge_dynamic_mask_amd", "libdma.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdma.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dma_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def dma():
    import doge_dynamic_mask_amd as m
    return m.lib()


def test_exports_every_declared_symbol(dma):
    names = declared_functions()
    assert set(names) >= {"dma_dt", "dma_select", "dma_attn_fwd", "dma_decode",
                          "dma_decode_workspace_bytes", "dma_status_str", "dma_version"}
    for n in names:
        assert hasattr(dma, n), n
    import doge_dynamic_mask_amd as m
    assert set(m.EXPORTS) == set(names)


def test_version_and_status_strings(dma):
    assert dma.dma_version() == 100
    for s in range(-6, 1):
        assert dma.dma_status_str(s)
    assert dma.dma_status_str(-99) == b"unknown status"


# Non-null, never-dereferenced stand-ins: every call below must fail host-side
# validation before it could touch them.
FAKE = ctypes.c_void_p(0x1000)
FAKE2 = ctypes.c_void_p(0x2000)


def test_dt_validation(dma):
    ok = dict(V=FAKE, W=FAKE, bias=None, A=FAKE, dtype=1, B=1, S=8, Hkv=2, d=64, out=FAKE, ld=8, pos=None)

    def call(**kw):
        a = {**ok, **kw}
        return dma.dma_dt(a["V"], a["W"], a["bias"], a["A"], a["dtype"], a["B"], a["S"], a["Hkv"], a["d"],
                          a["out"], a["ld"], a["pos"], None)
    assert call(V=None) == -1
    assert call(out=None) == -1
    assert call(A=None) == -1
    assert call(dtype=7) == -3
    assert call(B=0) == -2
    assert call(ld=4) == -2
    assert call(d=96) == -4
    assert call(Hkv=17) == -4
    assert call(V=ctypes.c_void_p(0x1004)) == -4  # misaligned


def test_select_validation(dma):
    assert dma.dma_select(None, None, 1, 1, 8, 2, FAKE, FAKE, None) == -1
    assert dma.dma_select(FAKE, None, 1, 1, 8, 0, FAKE, FAKE, None) == -2
    assert dma.dma_select(FAKE, None, 0, 1, 8, 2, FAKE, FAKE, None) == -2
    assert dma.dma_select(FAKE, None, 1, 1, 0, 2, FAKE, FAKE, None) == -2
    # one workgroup per (batch, kv head, 64-row chunk) on a 1-D grid: more
    # than 2^31 - 8 of them is refused before any launch
    assert dma.dma_select(FAKE, None, 65536, 512, 4096, 2, FAKE, FAKE, None) == -4
    assert dma.dma_select_window(FAKE, None, 65536, 512, 4096, 2, 64, FAKE, FAKE, None) == -4


def test_attn_validation(dma):
    def call(Q=FAKE, dtype=1, B=1, S=8, Hq=4, Hkv=2, d=64, w=4, O=FAKE2):
        return dma.dma_attn_fwd(Q, FAKE, FAKE, dtype, FAKE, FAKE, FAKE, None, B, S, Hq, Hkv, d, w, O, None)
    assert call(Q=None) == -1
    assert call(O=None) == -1
    assert call(dtype=2) == -3
    assert call(Hq=3) == -2
    assert call(w=0) == -2
    assert call(d=32) == -4
    assert call(Hq=258, Hkv=2) == -4


def test_decode_validation(dma):
    need = dma.dma_decode_workspace_bytes(4, 2048, 8, 2, 128, 256)
    assert need > 0
    assert dma.dma_decode_workspace_bytes(0, 2048, 8, 2, 128, 256) == 0

    def call(ws=FAKE2, nbytes=need, cache_lens=FAKE, d=128, Hq=8, Hkv=2):
        return dma.dma_decode(FAKE, FAKE, FAKE, 1, FAKE, cache_lens, 4, 2048, Hq, Hkv, d, 256,
                              FAKE, None, ws, nbytes, None)
    assert call(cache_lens=None) == -1
    assert call(ws=None) == -5
    assert call(nbytes=need - 1) == -5
    assert call(Hq=7) == -2
    assert call(Hq=64, Hkv=2) == -4
    assert call(d=80) == -4


def test_decode_state_validation(dma):
    nst = dma.dma_decode_state_bytes(2, 2, 128, 64)
    nws = dma.dma_decode_step_workspace_bytes(2, 8, 2, 128, 64)
    assert nst > 0 and nws > 0
    assert dma.dma_decode_state_bytes(2, 2, 96, 64) == 0
    assert dma.dma_decode_step_workspace_bytes(2, 7, 2, 128, 64) == 0

    def init(Kc=FAKE, dtype=1, state=FAKE2, sb=nst, ws=FAKE2, wb=nws, d=128, w=64):
        return dma.dma_decode_state_init(Kc, FAKE, dtype, FAKE, FAKE, 2, 100, 2, d, w, state, sb, ws, wb, None)
    assert init(Kc=None) == -1
    assert init(state=None) == -1
    assert init(dtype=5) == -3
    assert init(dtype=0) == -4        # float32 K/V: the state path is bf16 only
    assert init(w=0) == -2
    assert init(d=80) == -4
    assert init(sb=nst - 1) == -5
    assert init(ws=None) == -5

    def step(q=FAKE, dtype=1, Hq=8, sb=nst, wb=nws, out=FAKE2):
        return dma.dma_decode_step(q, FAKE, FAKE, dtype, FAKE, 2, Hq, 2, 128, 64, FAKE2, sb, out, FAKE2, wb, None)
    assert step(q=None) == -1
    assert step(out=None) == -1
    assert step(dtype=0) == -4
    assert step(Hq=7) == -2
    assert step(Hq=64) == -4
    assert step(sb=nst - 1) == -5
    assert step(wb=nws - 1) == -5
    assert step(q=ctypes.c_void_p(0x1008)) == -4
    assert dma.dma_decode_state_kept(None, nst, 2, 2, 128, 64, FAKE, None, None) == -1
    assert dma.dma_decode_state_kept(FAKE, nst - 1, 2, 2, 128, 64, FAKE, None, None) == -5


def test_qk_norm_rope_validation(dma):
    def call(Q=FAKE, dtype=1, wq=FAKE, eps=1e-6, theta=10000.0, B=2, S=8, Hq=4, Hkv=2, d=64, Qo=FAKE2):
        return dma.dma_qk_norm_rope(Q, FAKE, dtype, wq, FAKE, eps, theta, None, B, S, Hq, Hkv, d, Qo, FAKE2, None)
    assert call(Q=None) == -1
    assert call(wq=None) == -1
    assert call(Qo=None) == -1
    assert call(dtype=3) == -3
    assert call(B=0) == -2
    assert call(S=0) == -2
    assert call(eps=-1.0) == -2
    assert call(eps=float("nan")) == -2
    assert call(theta=1.0) == -2
    assert call(B=65536, S=65536) == -2       # more tokens than an int32 counts
    assert call(d=96) == -4
    assert call(Qo=ctypes.c_void_p(0x2008)) == -4

    def pro(V=FAKE, W=FAKE, A=FAKE, dt=FAKE2, Hkv=2, d=64, Q=FAKE):
        return dma.dma_prologue(Q, FAKE, V, 1, FAKE, FAKE, 1e-6, 10000.0, None, W, None, A, 2, 8, 4, Hkv, d,
                                FAKE2, FAKE2, dt, None)
    assert pro(V=None) == -1
    assert pro(A=None) == -1
    assert pro(dt=None) == -1
    assert pro(Q=None) == -1
    assert pro(Hkv=17) == -4
    assert pro(W=ctypes.c_void_p(0x1004)) == -4


def test_bwd_validation(dma):
    need = dma.dma_attn_bwd_workspace_bytes(2, 64, 8, 2, 64, 16)
    assert need > 0 and dma.dma_attn_bwd_workspace_bytes(2, 64, 7, 2, 64, 16) == 0

    def call(Q=FAKE, dtype=1, Hq=8, Hkv=2, d=64, ws=FAKE2, nb=need, dO=FAKE):
        return dma.dma_attn_bwd(Q, FAKE, FAKE, dtype, FAKE, FAKE, FAKE, None, dO, 2, 64, Hq, Hkv, d, 16,
                                FAKE2, FAKE2, FAKE2, FAKE2, ws, nb, None)
    assert call(Q=None) == -1
    assert call(dO=None) == -1
    assert call(dtype=4) == -3
    assert call(dtype=0) == -4        # float32: the backward is bf16 only
    assert call(Hq=7) == -2
    assert call(Hq=6, Hkv=2) == -4    # G = 3 does not divide the 64-pair tiles
    assert call(Hq=32, Hkv=2) == -4   # G = 16
    assert call(d=96) == -4
    assert call(ws=None) == -5
    assert call(nb=need - 1) == -5
    nd = dma.dma_dt_bwd_workspace_bytes(2, 64, 4, 64)
    assert nd > 0

    def dcall(V=FAKE, dW=FAKE2, Hkv=4, d=64, ws=FAKE2, nb=nd):
        return dma.dma_dt_bwd(V, FAKE, None, FAKE, 1, FAKE, 2, 64, Hkv, d, None, dW, None, FAKE2, ws, nb, None)
    assert dcall(V=None) == -1
    assert dcall(dW=None) == -1
    assert dcall(Hkv=17) == -4
    assert dcall(Hkv=16, d=128) == -4  # W would not fit the workgroup's LDS
    assert dcall(ws=None) == -5
    assert dcall(V=ctypes.c_void_p(0x1002)) == -4  # misaligned


def test_window_validation(dma):
    assert dma.dma_select_window(None, None, 1, 1, 8, 2, 4, FAKE, FAKE, None) == -1
    assert dma.dma_select_window(FAKE, None, 1, 1, 8, 2, 0, FAKE, FAKE, None) == -2
    assert dma.dma_select_window(FAKE, None, 1, 1, 8, 0, 4, FAKE, FAKE, None) == -2

    def call(Q=FAKE, dtype=1, Hq=4, Hkv=2, d=64, win=16, O=FAKE2):
        return dma.dma_attn_window_fwd(Q, FAKE, FAKE, dtype, FAKE, FAKE, FAKE, None, 1, 64, Hq, Hkv, d, 8, win, O,
                                       None)
    assert call(Q=None) == -1
    assert call(O=None) == -1
    assert call(dtype=2) == -3
    assert call(dtype=0) == -4
    assert call(win=0) == -2
    assert call(Hq=6, Hkv=2) == -4
    assert call(d=80) == -4


def test_cdmoe_validation(dma):
    assert dma.dma_cdmoe_logits(None, FAKE, 1, 4, 64, 8, FAKE2, None) == -1
    assert dma.dma_cdmoe_logits(FAKE, FAKE, 0, 4, 64, 8, FAKE2, None) == -4    # bf16 only
    assert dma.dma_cdmoe_logits(FAKE, FAKE, 1, 4, 60, 8, FAKE2, None) == -4    # H % 32
    assert dma.dma_cdmoe_logits(FAKE, FAKE, 1, 4, 64, 300, FAKE2, None) == -4  # nk > 256
    assert dma.dma_cdmoe_route(None, 4, 16, 4, FAKE, FAKE2, None) == -1
    assert dma.dma_cdmoe_route(FAKE, 4, 16, 17, FAKE, FAKE2, None) == -2       # k > nk
    assert dma.dma_cdmoe_route(FAKE, 4, 256, 129, FAKE, FAKE2, None) == -4     # k > 128
    assert dma.dma_cdmoe_experts(FAKE, FAKE, FAKE, 1, FAKE, None, 4, 512, 8, 4, FAKE2, None) == -1
    assert dma.dma_cdmoe_experts(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 4, 500, 8, 4, FAKE2, None) == -4
    assert dma.dma_cdmoe_experts(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 4, 512, 16, 129, FAKE2, None) == -4


def test_generic_workspace_query(dma):
    """dma_workspace_bytes(op, ...) dispatches to the per-operation queries;
    the operations without scratch report 0; unknown ops and bad sizes give
    (size_t)-1."""
    bad = ctypes.c_size_t(-1).value
    dma.dma_workspace_bytes.restype = ctypes.c_size_t
    B, S, Hq, Hkv, d, w = 4, 2048, 8, 2, 128, 256
    for op in (0, 1, 2):
        assert dma.dma_workspace_bytes(op, B, S, Hq, Hkv, d, w) == 0
    assert dma.dma_workspace_bytes(3, B, S, Hq, Hkv, d, w) == dma.dma_decode_workspace_bytes(B, S, Hq, Hkv, d, w)
    assert dma.dma_workspace_bytes(4, B, S, Hq, Hkv, d, w) == dma.dma_decode_step_workspace_bytes(B, Hq, Hkv, d, w)
    assert dma.dma_workspace_bytes(5, B, S, Hq, Hkv, 64, w) == dma.dma_attn_bwd_workspace_bytes(B, S, Hq, Hkv, 64, w)
    assert dma.dma_workspace_bytes(6, B, S, Hq, Hkv, 64, w) == dma.dma_dt_bwd_workspace_bytes(B, S, Hkv, 64)
    for op in (3, 4, 5, 6):
        assert dma.dma_workspace_bytes(op, B, S, Hq, Hkv, d, w) > 0
    assert dma.dma_workspace_bytes(7, B, S, Hq, Hkv, d, w) == bad
    assert dma.dma_workspace_bytes(-1, B, S, Hq, Hkv, d, w) == bad
    assert dma.dma_workspace_bytes(3, 0, S, Hq, Hkv, d, w) == bad
    assert dma.dma_workspace_bytes(0, B, S, 7, Hkv, d, w) == bad       # Hq % Hkv != 0
    assert dma.dma_workspace_bytes(5, B, S, Hq, Hkv, 96, w) == bad     # head_dim the backward rejects
    import doge_dynamic_mask_amd as m
    assert m.workspace_bytes(m.OP_DECODE, B, S, Hq, Hkv, d, w) == dma.dma_decode_workspace_bytes(B, S, Hq, Hkv, d, w)
    with pytest.raises(ValueError):
        m.workspace_bytes(9, B, S, Hq, Hkv, d, w)


def test_decode_noalloc_validation(dma):
    """The allocation-free decode rejects bad arguments, and sizes whose
    workspace exceeds its 16 MiB static array, before any HIP call."""
    def call(q=FAKE, cache_lens=FAKE, dtype=1, B=4, Lmax=2048, Hq=8, Hkv=2, d=128, w=256, out=FAKE2):
        return dma.dma_decode_noalloc(q, FAKE, FAKE, dtype, FAKE, cache_lens, B, Lmax, Hq, Hkv, d, w, out, None,
                                      None)
    assert call(q=None) == -1
    assert call(cache_lens=None) == -1
    assert call(out=None) == -1
    assert call(dtype=9) == -3
    assert call(Hq=7) == -2
    assert call(w=0) == -2
    assert call(d=80) == -4
    assert call(Hq=64, Hkv=2) == -4
    # the decode workload's workspace fits; a 64k-position cache with w = 8192 does not
    assert dma.dma_decode_workspace_bytes(64, 16384, 8, 2, 128, 2048) <= 16 << 20
    assert dma.dma_decode_workspace_bytes(64, 65536, 16, 2, 128, 8192) > 16 << 20
    assert call(B=64, Lmax=65536, Hq=16, Hkv=2, d=128, w=8192) == -5

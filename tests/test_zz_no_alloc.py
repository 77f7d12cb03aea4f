"""dma_decode_noalloc (workspace in the library's static device array) against
dma_decode (caller's workspace), through the C ABI: two calls in a row, the
second smaller than the first, then a float32 call.  Kept sets must be
identical and outputs within the parity bar (2e-2 for bf16, 1e-4 for
float32; the bf16 kernels are deterministic, so their outputs are compared
bit for bit, while the float32 path sums its waves' partial products with
LDS atomics, whose order varies from run to run).  Sizes whose workspace
exceeds the array are rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

DMA_ERR_WORKSPACE = -5


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _decode_inputs(wl, B, S, seed):
    import doge_dynamic_mask_amd as dma
    inp = si.make_inputs(wl, seed=seed, B=B, S=S)
    q, Kc, Vc = to_dev(inp["q"]), to_dev(inp["Kc"]), to_dev(inp["Vc"])
    dtc = dma.dt(Vc, to_dev(inp["W"]), to_dev(inp["A"]), to_dev(inp["bias"]))
    rng = np.random.default_rng(seed + 1)
    lens = rng.integers(1, S, size=B, endpoint=True).astype(np.int32)
    lens[0] = S
    return q, Kc, Vc, dtc, to_dev(lens)


def _both(q, Kc, Vc, dtc, lens, w):
    import doge_dynamic_mask_amd as dma
    L = dma.lib()
    B, Hq, d = q.shape
    Lmax, Hkv = Kc.shape[1], Kc.shape[2]
    code = dma.BF16 if q.dtype == torch.bfloat16 else dma.F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = int(L.dma_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, w))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    out_ref, kept_ref = torch.empty_like(q), torch.empty((B, Hkv, w), dtype=torch.int32, device=q.device)
    out_na, kept_na = torch.full_like(q, float("nan")), torch.full((B, Hkv, w), -7, dtype=torch.int32,
                                                                   device=q.device)
    st = L.dma_decode(_ptr(q), _ptr(Kc), _ptr(Vc), code, _ptr(dtc), _ptr(lens), B, Lmax, Hq, Hkv, d, w,
                      _ptr(out_ref), _ptr(kept_ref), _ptr(ws), nbytes, stream)
    assert st == 0, st
    st = L.dma_decode_noalloc(_ptr(q), _ptr(Kc), _ptr(Vc), code, _ptr(dtc), _ptr(lens), B, Lmax, Hq, Hkv, d, w,
                              _ptr(out_na), _ptr(kept_na), stream)
    assert st == 0, st
    torch.cuda.synchronize()
    return (to_host(out_ref), to_host(kept_ref)), (to_host(out_na), to_host(kept_na))


def test_noalloc_decode_matches_decode_two_calls():
    # first: the decode workload (B64, 16384 cached positions, Hq8 Hkv2 d128 w2048, ~10 MiB of workspace)
    wl = si.WORKLOADS["decode"]
    args = _decode_inputs(wl, wl.B, wl.S, seed=501)
    (o_ref, k_ref), (o_na, k_na) = _both(*args, wl.w)
    np.testing.assert_array_equal(k_na, k_ref)
    np.testing.assert_array_equal(o_na, o_ref)
    assert np.isfinite(o_na).all()
    del args
    # second, smaller: fewer batches, a shorter cache, d = 64, other heads and w
    small = si.Workload("na_small", "bf16", 5, 4, 1, 3000, 64, 700, decode=True, seed=502)
    args = _decode_inputs(small, small.B, small.S, seed=502)
    (o_ref, k_ref), (o_na, k_na) = _both(*args, small.w)
    np.testing.assert_array_equal(k_na, k_ref)
    np.testing.assert_array_equal(o_na, o_ref)
    assert np.isfinite(o_na).all()
    # float32 values through the same array
    f32 = si.Workload("na_f32", "f32", 3, 4, 2, 900, 128, 300, decode=True, seed=503)
    args = _decode_inputs(f32, f32.B, f32.S, seed=503)
    (o_ref, k_ref), (o_na, k_na) = _both(*args, f32.w)
    np.testing.assert_array_equal(k_na, k_ref)
    assert np.isfinite(o_na).all()
    assert np.abs(o_na - o_ref).max() <= 1e-4


def test_noalloc_decode_rejects_oversized_workspace():
    import doge_dynamic_mask_amd as dma
    L = dma.lib()
    B, Lmax, Hq, Hkv, d, w = 64, 65536, 16, 2, 128, 8192
    assert L.dma_decode_workspace_bytes(B, Lmax, Hq, Hkv, d, w) > dma.DECODE_NOALLOC_MAX_WORKSPACE
    fake = ctypes.c_void_p(0x1000)
    st = L.dma_decode_noalloc(fake, fake, fake, dma.BF16, fake, fake, B, Lmax, Hq, Hkv, d, w, fake, None, None)
    assert st == DMA_ERR_WORKSPACE

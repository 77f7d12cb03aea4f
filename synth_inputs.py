"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds random draws and the storage conversion of those draws to
bfloat16 only -- none of the method's arithmetic.  Both the HIP path and the
CPU oracle receive the very same arrays from here.

Workloads (shapes echo the Doge pages: S=2048 is the SFT context length of the
Doge-320M card's training table, keep_window_size=2048 is the DogeConfig
default, Hq=8 / d=128 are the DogeConfig defaults for heads and head_dim):

  tiny   fp32  B1 Hq2  Hkv1 S256   d64  w64
  c2     bf16  B4 Hq8  Hkv4 S2048  d64  w512
  long   bf16  B1 Hq16 Hkv8 S8192  d128 w2048
  decode bf16  B64 (one query each) cache 16384, Hq8 Hkv2 d128 w2048
  padded bf16  B2 Hq16 Hkv4 S32768 d128 w2048, lengths ~ U[16384, 32768]

Draw order per workload, from numpy's PCG64 seeded with ``seed``:
A ~ U(-2, 2) with exact zeros redrawn, W ~ N(0, 0.02^2), bias = 0, the padded
lengths (integers, inclusive bounds), then Q, K, V ~ N(0, 1) (decode: q, Kc,
Vc).  Draws are float32 and are rounded once to bfloat16 (nearest-even) for
the bf16 workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    S: int              # sequence length (prefill) or cache length (decode)
    d: int
    w: int
    decode: bool = False
    pad_lo: int = 0     # padded workloads: lengths ~ U[pad_lo, pad_hi]
    pad_hi: int = 0
    seed: int = 0
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", "f32", 1, 2, 1, 256, 64, 64, seed=1001,
                     note="DMA fwd tiny fp32, causal, no padding"),
    "c2": Workload("c2", "bf16", 4, 8, 4, 2048, 64, 512, seed=1002,
                   note="DMA prefill bf16, causal"),
    "long": Workload("long", "bf16", 1, 16, 8, 8192, 128, 2048, seed=1003,
                     note="DMA prefill bf16 long, causal"),
    "decode": Workload("decode", "bf16", 64, 8, 2, 16384, 128, 2048, decode=True, seed=1004,
                       note="DMA decode bf16, one query per batch over a 16384 cache"),
    "padded": Workload("padded", "bf16", 2, 16, 4, 32768, 128, 2048, pad_lo=16384,
                       pad_hi=32768, seed=1005,
                       note="DMA prefill bf16, right padding"),
}


def to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x40).astype(np.uint32), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else to_bf16_bits(x)


def _draw_A(rng, n):
    A = rng.uniform(-2.0, 2.0, size=n).astype(np.float32)
    while (A == 0).any():
        z = A == 0
        A[z] = rng.uniform(-2.0, 2.0, size=int(z.sum())).astype(np.float32)
    return A


def make_inputs(wl: Workload, seed: int | None = None, *, B=None, S=None):
    """All inputs of a workload as NumPy arrays (float32, or uint16 bf16 bits).

    ``B``/``S`` shrink a workload for quick tests without changing its draw
    recipe.  Prefill keys: Q, K, V, W, bias, A, seqlens (None when unpadded).
    Decode keys: q, Kc, Vc, W, bias, A, cache_lens.
    """
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B = wl.B if B is None else B
    S = wl.S if S is None else S
    Hq, Hkv, d = wl.Hq, wl.Hkv, wl.d
    A = _draw_A(rng, Hkv)
    W = rng.normal(0.0, 0.02, size=(Hkv, Hkv * d)).astype(np.float32)
    out = {"A": A, "W": _store(W, wl.dtype), "bias": _store(np.zeros(Hkv, np.float32), wl.dtype)}
    lens = None
    if wl.pad_hi:
        lo, hi = min(wl.pad_lo, S), min(wl.pad_hi, S)
        lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    if wl.decode:
        out["q"] = _store(rng.standard_normal((B, Hq, d), dtype=np.float32), wl.dtype)
        out["Kc"] = _store(rng.standard_normal((B, S, Hkv, d), dtype=np.float32), wl.dtype)
        out["Vc"] = _store(rng.standard_normal((B, S, Hkv, d), dtype=np.float32), wl.dtype)
        out["cache_lens"] = lens if lens is not None else np.full(B, S, np.int32)
    else:
        out["Q"] = _store(rng.standard_normal((B, S, Hq, d), dtype=np.float32), wl.dtype)
        out["K"] = _store(rng.standard_normal((B, S, Hkv, d), dtype=np.float32), wl.dtype)
        out["V"] = _store(rng.standard_normal((B, S, Hkv, d), dtype=np.float32), wl.dtype)
        out["seqlens"] = lens
    return out


def make_qkv(B, S, Hq, Hkv, d, dtype, seed):
    """Q [B,S,Hq,d], K/V [B,S,Hkv,d] ~ N(0,1), stored as float32 or bf16 bits."""
    rng = np.random.default_rng(seed)
    Q = _store(rng.standard_normal((B, S, Hq, d), dtype=np.float32), dtype)
    K = _store(rng.standard_normal((B, S, Hkv, d), dtype=np.float32), dtype)
    V = _store(rng.standard_normal((B, S, Hkv, d), dtype=np.float32), dtype)
    return Q, K, V


def make_dt(shape, kind: str, seed: int) -> np.ndarray:
    """Synthetic dt (float32, >= 0) for selection and attention parity cases.

    kinds:
      lognormal  continuous positive values, few exact ties
      dyadic     m * 2^-10 with integer m < 2^13: many exact ties
      const      every value 1.0 (all keys tie)
      few        values from a set of 5: heavy ties
      wide       log-uniform over [2^-20, 2^20]
      shared     2^18 + U(0, 4): a large dt common to every key, so the
                 scores' differences come from q.k and a small spread of dt
      spiky      lognormal with one key in 500 raised 10^6-fold: a few keys
                 far above the rest, easily missed by a sample of positions
      rising     position / n + U(0, 0.05) along the last axis: the largest
                 keys are the latest ones
    """
    rng = np.random.default_rng(seed)
    if kind == "lognormal":
        x = rng.lognormal(0.0, 0.8, size=shape)
    elif kind == "dyadic":
        x = rng.integers(0, 1 << 13, size=shape) * 2.0 ** -10
    elif kind == "const":
        x = np.ones(shape)
    elif kind == "few":
        x = rng.choice(np.array([0.25, 0.5, 1.0, 1.5, 3.0]), size=shape)
    elif kind == "wide":
        x = 2.0 ** rng.uniform(-20.0, 20.0, size=shape)
    elif kind == "shared":
        x = 2.0 ** 18 + rng.uniform(0.0, 4.0, size=shape)
    elif kind == "spiky":
        x = rng.lognormal(0.0, 0.8, size=shape)
        x = np.where(rng.uniform(size=shape) < 1.0 / 500, x * 1e6, x)
    elif kind == "rising":
        n = shape[-1]
        x = np.arange(n) / n + rng.uniform(0.0, 0.05, size=shape)
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(x, dtype=np.float32)


def make_lengths(B, lo, hi, seed) -> np.ndarray:
    """Right-padding lengths ~ U[lo, hi] (inclusive)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def make_norm_weights(d, dtype, seed):
    """q_norm and k_norm weights, each [d] ~ U(0.5, 1.5), stored as float32 or bf16
    bits (RMSNorm weights start at ones; trained ones spread around that)."""
    rng = np.random.default_rng(seed)
    wq = rng.uniform(0.5, 1.5, size=d).astype(np.float32)
    wk = rng.uniform(0.5, 1.5, size=d).astype(np.float32)
    return _store(wq, dtype), _store(wk, dtype)


def make_positions(B, S, kind, seed) -> np.ndarray:
    """Token positions [B, S] int32.

    kinds:
      offset  s + o_b with o_b ~ U[0, 2^20]: a chunk after o_b cached tokens
      large   independent ~ U[0, 2^30): angles far from the first turns
    """
    rng = np.random.default_rng(seed)
    if kind == "offset":
        o = rng.integers(0, 1 << 20, size=(B, 1), endpoint=True)
        p = o + np.arange(S)[None, :]
    elif kind == "large":
        p = rng.integers(0, 1 << 30, size=(B, S))
    else:
        raise ValueError(kind)
    return np.ascontiguousarray(p, dtype=np.int32)


def make_cdmoe(T, H, nk, dtype, seed):
    """CDMoE inputs: hidden states h [T, H] ~ N(0, 1), router_gate [2*nk, H],
    down_embed and up_embed [nk*nk, H] ~ N(0, 0.02^2) (the DogeConfig
    initializer_range), stored as float32 or bf16 bits."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, H), dtype=np.float32)
    router = rng.normal(0.0, 0.02, size=(2 * nk, H)).astype(np.float32)
    down = rng.normal(0.0, 0.02, size=(nk * nk, H)).astype(np.float32)
    up = rng.normal(0.0, 0.02, size=(nk * nk, H)).astype(np.float32)
    return _store(h, dtype), _store(router, dtype), _store(down, dtype), _store(up, dtype)

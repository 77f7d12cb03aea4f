"""Helpers for the GPU parity tests: move seeded NumPy inputs to the device and back."""
import numpy as np
import torch

import synth_inputs as si

DEV = "cuda:0"


def to_dev(x):
    """NumPy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    t = torch.from_numpy(x)
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def to_host(t):
    """Device tensor -> NumPy (bf16 -> float32 values, others unchanged)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return si.bf16_bits_to_f32(t.view(torch.uint16).numpy())
    return t.numpy()


def host_f64(x):
    """NumPy input (float32 or bf16 bits) -> float64 values."""
    return (si.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).astype(np.float64)


def sample_rows(B, Hkv, S, seqlens, n, seed, w=None):
    """(b, g, i) rows: edges (first rows, the w boundary, the last valid rows,
    padded rows) plus n random valid rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        L = S if seqlens is None else int(seqlens[b])
        for g in range(Hkv):
            edges = [0, 1, L - 1, L - 2, S - 1]
            if w is not None:
                edges += [w - 2, w - 1, w, w + 1]
            for i in edges:
                if 0 <= i < S:
                    rows.add((b, g, i))
    for _ in range(n):
        b = int(rng.integers(B))
        L = S if seqlens is None else int(seqlens[b])
        rows.add((b, int(rng.integers(Hkv)), int(rng.integers(L))))
    return np.array(sorted(rows), dtype=np.int32)

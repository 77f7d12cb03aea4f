"""Benchmark of the DMA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--extra]

One step = the whole hot path over one batch of synthetic input:
  prefill  B=4 Hq=8 Hkv=4 S=2048 d=64 w=512 bf16  (dma_dt -> dma_select -> dma_attn_fwd)
  decode   B=64 Hq=8 Hkv=2 d=128 w=2048, 16384 cached positions
           (dma_dt appends the new token's dt, then dma_decode)
A 512 MiB read before each decode evicts the kept K/V rows from the caches
(with clean lines, so no write-back traffic lands on the decode), so decode
moves its bytes from HBM; the eviction is outside the timed kernels.

Printed: ONE JSON line.  value = prefill kept-key TFLOP/s (kept (query, key)
pairs x 4*d flop over the GPU time of the three prefill kernels, replayed as
one HIP graph); the decode GB/s (algorithmic bytes over dma_decode's GPU
time) rides along under "decode".  ms_per_step = prefill + decode GPU time of
one step (the cache flush between them is excluded); the wall-clock time per
step including the flush is reported too.  Times come from HIP events
recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth_inputs as si  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak


def kept_flops(B, Hq, S, d, w, seqlens=None):
    """Sum over query heads and valid rows of 4*d*min(valid keys, w)."""
    total = 0
    for b in range(B):
        L = S if seqlens is None else int(seqlens[b])
        i = np.arange(L, dtype=np.int64)
        total += int(np.minimum(i + 1, w).sum()) * Hq
    return total * 4 * d


def decode_bytes(B, Hq, Hkv, d, w, lens, esize=2):
    """dt of every cached position + K/V rows of the kept positions + q + out."""
    total = 0
    for L in lens:
        total += Hkv * (int(L) * 4 + min(int(L), w) * 2 * d * esize) + 2 * Hq * d * esize
    return total


def to_dev(x, dev):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.view(torch.bfloat16) if x.dtype == np.uint16 else t).to(dev)


def cpu_baseline(pre_inp, wl_p, min_seconds=10.0):
    """The oracle (plain C, fp64, OpenMP) timed on the host: full prefill of
    the same batch (dt, select, attention over every row), repeated until
    min_seconds have passed.  Reported in the metric's unit (kept-key TFLOP/s)."""
    import oracle
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    flops = kept_flops(wl_p.B, wl_p.Hq, wl_p.S, wl_p.d, wl_p.w)
    reps, t0 = 0, time.perf_counter()
    while True:
        dt = oracle.dt(pre_inp["V"], pre_inp["W"], pre_inp["bias"], pre_inp["A"])
        dt32 = dt.astype(np.float32)
        oracle.select(dt32, wl_p.w)
        oracle.attn(pre_inp["Q"], pre_inp["K"], pre_inp["V"], dt32, wl_p.w)
        reps += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    el = time.perf_counter() - t0
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full prefill of the same batch (dt + select + attention, every row), "
                      f"{reps} repetitions in {el:.1f} s, fp64"}


def prefill_breakdown(dma, name, dev, reps=10):
    """Per-kernel GPU time of one prefill workload (graph replays between events)."""
    wl = si.WORKLOADS[name]
    inp = si.make_inputs(wl)
    Q, K, V = to_dev(inp["Q"], dev), to_dev(inp["K"], dev), to_dev(inp["V"], dev)
    W, A, bias = to_dev(inp["W"], dev), to_dev(inp["A"], dev), to_dev(inp["bias"], dev)
    seq = None if inp["seqlens"] is None else to_dev(inp["seqlens"], dev)
    dt = torch.empty((wl.B, wl.Hkv, wl.S), dtype=torch.float32, device=dev)
    tau, tie = torch.empty_like(dt), torch.empty(dt.shape, dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    fns = {"dt": lambda: dma.dt(V, W, A, bias, out=dt),
           "select": lambda: dma.select(dt, wl.w, seq, tau=tau, tie=tie),
           "attn_fwd": lambda: dma.attn_fwd(Q, K, V, dt, tau, tie, wl.w, seq, out=O)}
    res = {}
    for n, f in fns.items():
        f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        res[n] = a.elapsed_time(b) / reps
    flops = kept_flops(wl.B, wl.Hq, wl.S, wl.d, wl.w, inp["seqlens"])
    tot = sum(res.values())
    return {"ms": {k: round(v, 5) for k, v in res.items()}, "kept_flops": flops,
            "tflops_prefill": round(flops / (tot * 1e-3) / 1e12, 2),
            "tflops_attn": round(flops / (res["attn_fwd"] * 1e-3) / 1e12, 2),
            "attn_frac_of_peak": round(flops / (res["attn_fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--other-configs", action="store_true",
                    help="also time the other prefill workloads (long, padded, tiny) per kernel")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the DMA hot path has no cross-GPU step in this build "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import doge_dynamic_mask_amd as dma
    dma.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl_p = si.WORKLOADS["c2"]
    wl_d = si.WORKLOADS["decode"]
    pre = si.make_inputs(wl_p)
    dec = si.make_inputs(wl_d)

    Q, K, V = to_dev(pre["Q"], dev), to_dev(pre["K"], dev), to_dev(pre["V"], dev)
    W, A, bias = to_dev(pre["W"], dev), to_dev(pre["A"], dev), to_dev(pre["bias"], dev)
    dt = torch.empty((wl_p.B, wl_p.Hkv, wl_p.S), dtype=torch.float32, device=dev)
    tau = torch.empty_like(dt)
    tie = torch.empty(dt.shape, dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)

    q, Kc, Vc = to_dev(dec["q"], dev), to_dev(dec["Kc"], dev), to_dev(dec["Vc"], dev)
    Wd, Ad, biasd = to_dev(dec["W"], dev), to_dev(dec["A"], dev), to_dev(dec["bias"], dev)
    lens = to_dev(dec["cache_lens"], dev)
    pos = lens - 1
    dt_cache = dma.dt(Vc, Wd, Ad, biasd)          # the cache's dt, built once (untimed)
    v_new = Vc[torch.arange(wl_d.B, device=dev), pos.long()].unsqueeze(1).contiguous()
    out = torch.empty_like(q)
    ws = torch.empty(dma.decode_workspace_bytes(wl_d.B, wl_d.S, wl_d.Hq, wl_d.Hkv, wl_d.d, wl_d.w),
                     dtype=torch.uint8, device=dev)
    flush_buf = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def evict():
        torch.sum(flush_buf, dim=0, out=flush_out)

    torch.cuda.synchronize()

    # Each stage is captured once into a HIP graph (the binding launches on
    # torch's current stream, which is the capture stream), so a replay costs
    # one launch and the events below time GPU work rather than Python.
    def g_dt():
        dma.dt(V, W, A, bias, out=dt)

    def g_select():
        dma.select(dt, wl_p.w, tau=tau, tie=tie)

    def g_attn():
        dma.attn_fwd(Q, K, V, dt, tau, tie, wl_p.w, out=O)

    def g_dt_append():
        dma.dt(v_new, Wd, Ad, biasd, out=dt_cache, out_pos=pos)

    def g_decode():
        dma.decode(q, Kc, Vc, dt_cache, lens, wl_d.w, out=out, workspace=ws)

    def capture(*fns):
        for f in fns:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in fns:
                f()
        torch.cuda.synchronize()
        return g

    G_pre = capture(g_dt, g_select, g_attn)
    G_dec = capture(g_dt_append, g_decode)
    single = {"dt": capture(g_dt), "select": capture(g_select), "attn_fwd": capture(g_attn),
              "dt_append": capture(g_dt_append), "decode": capture(g_decode)}

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(e=None):
        if e:
            e[0].record()
        G_pre.replay()
        if e:
            e[1].record()
        evict()
        if e:
            e[2].record()
        G_dec.replay()
        if e:
            e[3].record()

    for _ in range(args.warmup):
        step()
    evs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_pre = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    ms_dec = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    # Per-kernel average durations: REPS back-to-back replays of a one-kernel
    # graph between two events; the decode kernels run after a cache flush.
    REPS = 20
    avg = {}
    for n, g in single.items():
        if n in ("dt_append", "decode"):
            pairs = []
            for _ in range(REPS):
                evict()
                a, b = ev(), ev()
                a.record()
                g.replay()
                b.record()
                pairs.append((a, b))
            torch.cuda.synchronize()
            avg[n] = float(np.mean([a.elapsed_time(b) for a, b in pairs]))
        else:
            a, b = ev(), ev()
            a.record()
            for _ in range(REPS):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            avg[n] = a.elapsed_time(b) / REPS

    flops = kept_flops(wl_p.B, wl_p.Hq, wl_p.S, wl_p.d, wl_p.w)
    value = flops / (ms_pre * 1e-3) / 1e12
    dbytes = decode_bytes(wl_d.B, wl_d.Hq, wl_d.Hkv, wl_d.d, wl_d.w, dec["cache_lens"])
    dec_gbs = dbytes / (avg["decode"] * 1e-3) / 1e9
    attn_tflops = flops / (avg["attn_fwd"] * 1e-3) / 1e12

    line = {
        "metric": "DMA prefill kept-key TFLOP/s + decode GB/s, % of MI355X roofline",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_pre + ms_dec, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, N(0,0.02) dt_proj, A~U(-2,2))",
        "config": {
            "workload": "prefill B4 Hq8 Hkv4 S2048 d64 w512 (dt+select+attn) + decode B64 L16384 Hq8 Hkv2 "
                        "d128 w2048 (dt append + decode)",
            "prefill_kept_flops": flops,
            "decode_bytes": dbytes,
        },
        "roofline": {
            "bound": "mfma", "kernel": "dma_attn_fwd (attn_bf16_kernel<64>)",
            "achieved": round(attn_tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 5), "traffic": None,
        },
        "decode": {
            "value": round(dec_gbs, 2), "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
            "frac": round(dec_gbs / PEAK_HBM_GBS, 5),
        },
        "ms_prefill": round(ms_pre, 5),
        "ms_decode_step": round(ms_dec, 5),
        "kernel_ms_avg": {n: round(v, 5) for n, v in avg.items()},
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
    }
    if args.other_configs:
        line["other_configs"] = {n: prefill_breakdown(dma, n, dev) for n in ("long", "padded")}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pre, wl_p)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

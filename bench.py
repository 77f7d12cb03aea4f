"""Benchmark of the DMA forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--other-configs]
    python bench.py --copy-calibration     (a plain 256 MiB copy, for counter scaling)

One step = the whole hot path over one batch of synthetic input:
  prefill  B=4 Hq=8 Hkv=4 S=2048 d=64 w=512 bf16  (dma_dt -> dma_select -> dma_attn_fwd)
  decode   B=64 Hq=8 Hkv=2 d=128 w=2048, 16384 cached positions
           (dma_dt appends the new token's dt, then dma_decode)
A 512 MiB read before each decode evicts the kept K/V rows from the caches
(with clean lines, so no write-back traffic lands on the decode), so decode
moves its bytes from HBM; a 512 MiB read before the prefill does the same
for the prefill inputs.  The evictions are outside the timed kernels.

Printed: ONE JSON line.  value = prefill kept-key TFLOP/s (kept (query, key)
pairs x 4*d flop over the GPU time of the three prefill calls, launched back
to back); the decode GB/s (algorithmic bytes over dma_decode's GPU time)
rides along under "decode".  ms_per_step = prefill + decode GPU time of one
step (the cache evictions are excluded); the wall-clock time per step
including them is reported too.  Times come from HIP events recorded between
the calls on the stream the kernels run on; the prefill replayed as one HIP
graph is timed as well.
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

# HBM bytes per launch of the prefill attention kernel on this workload, from
# two rocprofv3 counter runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch), each scaled by copy_bytes / counter reading of a plain copy of
# known size (--copy-calibration); the runs and their readings are in
# profiles/dma_kernels_prefill_b4s2048_decode_b64l16384_hbm_counters.md.  The
# figure holds only for the attention source it was measured on: when the
# hash of those files differs, traffic is reported as null.
ATTN_TRAFFIC = {"bytes": 26108416,
                "sources_sha256": "dc85285bef52cf9b22312007b0b58318a801c0dbbb285bed3505c75e498a07df"}
ATTN_SOURCES = ("doge_dynamic_mask_amd/csrc/attn.hip", "doge_dynamic_mask_amd/csrc/common.hpp")
COPY_CAL_BYTES = 256 * 1024 * 1024


def sources_sha256(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_calibration():
    """Five plain device-to-device copies of COPY_CAL_BYTES, for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each": COPY_CAL_BYTES, "copies": 5}), flush=True)


def kept_flops(B, Hq, S, d, w, seqlens=None, win=None):
    """Sum over query heads and valid rows of 4*d*min(valid keys, w); with a
    sliding window of win positions a row has at most win valid keys."""
    total = 0
    for b in range(B):
        L = S if seqlens is None else int(seqlens[b])
        i = np.arange(L, dtype=np.int64)
        vis = i + 1 if win is None else np.minimum(i + 1, win)
        total += int(np.minimum(vis, w).sum()) * Hq
    return total * 4 * d


def decode_bytes(B, Hq, Hkv, d, w, lens, esize=2):
    """dt of every cached position + K/V rows of the kept positions + q + out."""
    total = 0
    for L in lens:
        total += Hkv * (int(L) * 4 + min(int(L), w) * 2 * d * esize) + 2 * Hq * d * esize
    return total


def decode_state_bytes_moved(B, Hq, Hkv, d, w, lens, esize=2):
    """Per incremental decode step: the selection key and K/V row of every kept
    slot, the new token's rows and dt, q and out."""
    total = 0
    for L in lens:
        n = min(int(L) + 1, w)
        total += Hkv * (n * (8 + 2 * d * esize) + 2 * d * esize + 4) + 2 * Hq * d * esize
    return total


def prologue_bytes(B, S, Hq, Hkv, d, esize=2):
    """Algorithmic HBM bytes of one dma_prologue call (in place): Q and K read
    and written once, V read once, dt written once, plus the norm weights and
    dt_proj's W, A and bias."""
    tok = B * S * ((2 * Hq + 3 * Hkv) * d * esize + Hkv * 4)
    return tok + (2 * d + Hkv * Hkv * d + Hkv) * esize + Hkv * 4


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
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": flops * reps / el / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"full prefill of the same batch (dt + select + attention, every row), "
                      f"{reps} repetitions in {el:.1f} s, fp64",
            "host": {"cpu_model": model, "visible_cpus": os.cpu_count()}}


def prefill_breakdown(dma, name, dev, evict, R=8, rounds=4):
    """Per-call GPU time of one prefill workload, timed like the main
    workload's calls: after an eviction, R back-to-back launches between two
    events, each on its own copy of the inputs (enough copies that every
    launch reads from HBM)."""
    wl = si.WORKLOADS[name]
    inp = si.make_inputs(wl)
    Q, K, V = to_dev(inp["Q"], dev), to_dev(inp["K"], dev), to_dev(inp["V"], dev)
    W, A, bias = to_dev(inp["W"], dev), to_dev(inp["A"], dev), to_dev(inp["bias"], dev)
    seq = None if inp["seqlens"] is None else to_dev(inp["seqlens"], dev)
    dt = torch.empty((wl.B, wl.Hkv, wl.S), dtype=torch.float32, device=dev)
    tau, tie = torch.empty_like(dt), torch.empty(dt.shape, dtype=torch.int32, device=dev)
    O = torch.empty_like(Q)
    dma.dt(V, W, A, bias, out=dt)
    dma.select(dt, wl.w, seq, tau=tau, tie=tie)
    first = (Q, K, V, dt, tau, tie)
    set_bytes = sum(t.numel() * t.element_size() for t in first)
    nsets = 1 + -(-300 * 2**20 // set_bytes)
    sets = [first] + [tuple(t.clone() for t in first) for _ in range(nsets - 1)]
    rot = [0]

    def nxt():
        rot[0] += 1
        return sets[rot[0] % nsets]

    def c_dt():
        s_ = nxt()
        dma.dt(s_[2], W, A, bias, out=s_[3])

    def c_select():
        s_ = nxt()
        dma.select(s_[3], wl.w, seq, tau=s_[4], tie=s_[5])

    def c_attn():
        s_ = nxt()
        dma.attn_fwd(*s_, wl.w, seq, out=O)

    res = {}
    for n, f in (("dt", c_dt), ("select", c_select), ("attn_fwd", c_attn)):
        pairs = []
        for _ in range(rounds):
            evict()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(R):
                f()
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        res[n] = float(np.mean([a.elapsed_time(b) for a, b in pairs])) / R
    del sets
    flops = kept_flops(wl.B, wl.Hq, wl.S, wl.d, wl.w, inp["seqlens"])
    tot = sum(res.values())
    return {"ms": {k: round(v, 5) for k, v in res.items()}, "kept_flops": flops, "input_copies": nsets,
            "tflops_prefill": round(flops / (tot * 1e-3) / 1e12, 2),
            "tflops_attn": round(flops / (res["attn_fwd"] * 1e-3) / 1e12, 2),
            "attn_frac_of_peak": round(flops / (res["attn_fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def window_breakdown(dma, dev, evict, win=4096, R=6, rounds=3):
    """The sliding-window variant on the long workload (B1 Hq16 Hkv8 S8192
    d128 w2048) with a window of `win` positions: per-call GPU time of
    dma_select_window and dma_attn_window_fwd, timed like the other calls
    (after an eviction, R launches each on its own copy of the inputs)."""
    wl = si.WORKLOADS["long"]
    inp = si.make_inputs(wl)
    Q, K, V = to_dev(inp["Q"], dev), to_dev(inp["K"], dev), to_dev(inp["V"], dev)
    dt = dma.dt(V, to_dev(inp["W"], dev), to_dev(inp["A"], dev), to_dev(inp["bias"], dev))
    tau, tie = dma.select_window(dt, wl.w, win)
    O = torch.empty_like(Q)
    first = (Q, K, V, dt, tau, tie)
    set_bytes = sum(t.numel() * t.element_size() for t in first)
    nsets = 1 + -(-300 * 2**20 // set_bytes)
    sets = [first] + [tuple(t.clone() for t in first) for _ in range(nsets - 1)]
    rot = [0]

    def nxt():
        rot[0] += 1
        return sets[rot[0] % nsets]

    def c_sel():
        s_ = nxt()
        dma.select_window(s_[3], wl.w, win, tau=s_[4], tie=s_[5])

    def c_attn():
        s_ = nxt()
        dma.attn_window_fwd(*s_, wl.w, win, out=O)

    res = {}
    for n, f in (("select_window", c_sel), ("attn_window_fwd", c_attn)):
        f()
        torch.cuda.synchronize()
        pairs = []
        for _ in range(rounds):
            evict()
            evict()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(R):
                f()
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        res[n] = float(np.mean([a.elapsed_time(b) for a, b in pairs])) / R
    del sets
    flops = kept_flops(wl.B, wl.Hq, wl.S, wl.d, wl.w, win=win)
    tot = sum(res.values())
    return {"workload": f"long (B1 Hq16 Hkv8 S8192 d128 w2048) with sliding_window {win}",
            "ms": {k: round(v, 5) for k, v in res.items()}, "kept_flops": flops,
            "tflops": round(flops / (tot * 1e-3) / 1e12, 2),
            "tflops_attn": round(flops / (res["attn_window_fwd"] * 1e-3) / 1e12, 2),
            "attn_frac_of_peak": round(flops / (res["attn_window_fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def cdmoe_breakdown(dma, dev, evict, T=8192, H=1024, nk=128, k=64, R=6, rounds=3):
    """CDMoE routed experts at the DogeConfig sizes (hidden 1024, 16384
    experts, 64 per token) for T tokens: per-call GPU time of the router
    product, the routing and the experts, each after an eviction."""
    h, router, down, up = (to_dev(x, dev) for x in si.make_cdmoe(T, H, nk, "bf16", seed=77))
    lg = dma.cdmoe_logits(h, router)
    idx, w = dma.cdmoe_route(lg, k)
    out = dma.cdmoe_experts(h, down, up, idx, w)
    calls = (("logits", lambda: dma.cdmoe_logits(h, router, out=lg)),
             ("route", lambda: dma.cdmoe_route(lg, k, idx=idx, weights=w)),
             ("experts", lambda: dma.cdmoe_experts(h, down, up, idx, w, out=out)))
    res = {}
    for n, f in calls:
        f()
        torch.cuda.synchronize()
        pairs = []
        for _ in range(rounds):
            evict()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(R):
                f()
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        res[n] = float(np.mean([a.elapsed_time(b) for a, b in pairs])) / R
    flops = 2.0 * T * H * 2 * nk
    gathered = T * k * H * 2 * 2          # down and up rows of every kept expert
    return {"workload": f"T{T} hidden {H}, {nk * nk} experts ({nk} keys per domain), {k} per token",
            "ms": {n: round(v, 5) for n, v in res.items()},
            "logits_tflops": round(flops / (res["logits"] * 1e-3) / 1e12, 2),
            "experts_gathered_gbs": round(gathered / (res["experts"] * 1e-3) / 1e9, 1),
            "note": "expert rows are gathered per token; the 64 MiB of tables stay in the last-level cache "
                    "after the first launch, so the gather rate exceeds HBM"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--other-configs", action="store_true",
                    help="also time the other prefill workloads (long, padded, tiny) per kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain copies of known size (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the DMA hot path here has no cross-GPU step "
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

    # The stages, each one call of the C ABI through the binding, which
    # launches on torch's current stream (the stream the events record on).
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

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # One step: evict, the three prefill calls back to back, evict, the two
    # decode calls.  The eviction keeps the GPU busy for ~0.14 ms while Python
    # enqueues what follows, so the events see GPU work rather than host
    # launch latency (host_enqueue_ms_per_step reports the enqueue time).
    PRE = (g_dt, g_select, g_attn)
    DEC = (g_dt_append, g_decode)
    host_ms = []

    def step(e=None):
        evict()
        h0 = time.perf_counter()
        if e:
            e[0].record()
        for f in PRE:
            f()
        if e:
            e[1].record()
        evict()
        if e:
            e[2].record()
        for f in DEC:
            f()
        if e:
            e[3].record()
        host_ms.append((time.perf_counter() - h0) * 1e3)

    for _ in range(args.warmup):
        step()
    evs = [[ev() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    host_ms.clear()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre_each = [e[0].elapsed_time(e[1]) for e in evs]
    dec_each = [e[2].elapsed_time(e[3]) for e in evs]
    ms_pre = float(np.mean(pre_each))
    ms_dec = float(np.mean(dec_each))

    # Average launch duration per call: after an eviction, R back-to-back
    # launches of one call between two events, ROUNDS times.  Each launch
    # reads its own copy of the inputs, rotating over enough copies that the
    # data read in between exceeds the 256 MB last-level cache, so that every
    # launch reads from HBM as in the steps above.
    R, ROUNDS = 12, 5
    NPRE = 20    # prefill input sets of ~16.4 MB
    NDEC = 4     # decode caches (~134 MB of kept rows each)
    pre_sets = [(Q, K, V, dt, tau, tie)] + [
        tuple(t.clone() for t in (Q, K, V, dt, tau, tie)) for _ in range(NPRE - 1)]
    dec_sets = [(Kc, Vc, dt_cache)] + [
        tuple(t.clone() for t in (Kc, Vc, dt_cache)) for _ in range(NDEC - 1)]
    rot = [0]

    def nxt(sets):
        rot[0] += 1
        return sets[rot[0] % len(sets)]

    def c_dt():
        _, _, v, d, _, _ = nxt(pre_sets)
        dma.dt(v, W, A, bias, out=d)

    def c_select():
        _, _, _, d, ta, ti = nxt(pre_sets)
        dma.select(d, wl_p.w, tau=ta, tie=ti)

    def c_attn():
        q_, k_, v_, d, ta, ti = nxt(pre_sets)
        dma.attn_fwd(q_, k_, v_, d, ta, ti, wl_p.w, out=O)

    def c_dt_append():
        dma.dt(v_new, Wd, Ad, biasd, out=nxt(dec_sets)[2], out_pos=pos)

    # The prologue upstream of dt (Q/K RMSNorm + rotary, then dt), in place on
    # the rotating input sets; timed after attn_fwd, whose inputs it rewrites.
    wq, wk = (to_dev(x, dev) for x in si.make_norm_weights(wl_p.d, wl_p.dtype, wl_p.seed + 7))

    def c_qk_norm_rope():
        q_, k_, _, _, _, _ = nxt(pre_sets)
        dma.qk_norm_rope(q_, k_, wq, wk, Q_out=q_, K_out=k_)

    def c_prologue():
        q_, k_, v_, d, _, _ = nxt(pre_sets)
        dma.prologue(q_, k_, v_, wq, wk, W, A, bias, Q_out=q_, K_out=k_, dt_out=d)

    # The backward of the prefill (attention gradients, then the dt chain's),
    # on the rotating input sets with one upstream gradient dO.
    dO = torch.randn_like(Q)
    ws_b = torch.empty(dma.attn_bwd_workspace_bytes(wl_p.B, wl_p.S, wl_p.Hq, wl_p.Hkv, wl_p.d, wl_p.w),
                       dtype=torch.uint8, device=dev)
    ws_db = torch.empty(dma.dt_bwd_workspace_bytes(wl_p.B, wl_p.S, wl_p.Hkv, wl_p.d), dtype=torch.uint8, device=dev)
    g_out = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V), torch.empty_like(dt))

    def c_attn_bwd():
        q_, k_, v_, d, ta, ti = nxt(pre_sets)
        dma.attn_bwd(q_, k_, v_, d, ta, ti, wl_p.w, dO, workspace=ws_b, out=g_out)

    def c_dt_bwd():
        _, _, v_, _, _, _ = nxt(pre_sets)
        dma.dt_bwd(v_, W, A, g_out[3], bias, dV=g_out[2], workspace=ws_db)

    def c_decode():
        kc, vc, dc = nxt(dec_sets)
        dma.decode(q, kc, vc, dc, lens, wl_d.w, out=out, workspace=ws)

    # The incremental decode: the state of the cache without its last token
    # (kept keys and their K/V rows, 137 MB), then steps that append that
    # token; three states in turn, so that each step reads its rows from HBM.
    NST = 3
    ar = torch.arange(wl_d.B, device=dev)
    k_last, v_last = Kc[ar, pos.long()].contiguous(), Vc[ar, pos.long()].contiguous()
    dt_last = dt_cache[ar, :, pos.long()].contiguous()
    states = [dma.decode_state_init(Kc, Vc, dt_cache, pos, wl_d.w) for _ in range(NST)]
    ws_step = torch.empty(dma.decode_step_workspace_bytes(wl_d.B, wl_d.Hq, wl_d.Hkv, wl_d.d, wl_d.w),
                          dtype=torch.uint8, device=dev)
    rot_st = [0]

    def c_decode_step():
        rot_st[0] += 1
        dma.decode_step(q, k_last, v_last, dt_last, states[rot_st[0] % NST], out=out, workspace=ws_step)

    calls = (("dt", c_dt), ("select", c_select), ("attn_fwd", c_attn),
             ("dt_append", c_dt_append), ("decode", c_decode), ("decode_step", c_decode_step),
             ("attn_bwd", c_attn_bwd), ("dt_bwd", c_dt_bwd),
             ("qk_norm_rope", c_qk_norm_rope), ("prologue", c_prologue))
    avg, host_launch_ms = {}, {}
    for n, f in calls:
        f()                         # the first launch of a kernel loads its code
        torch.cuda.synchronize()
        pairs = []
        hs = []
        for _ in range(ROUNDS):
            evict()
            evict()                 # ~0.28 ms for the host to enqueue the R launches
            a, b = ev(), ev()
            a.record()
            h0 = time.perf_counter()
            for _ in range(R):
                f()
            hs.append((time.perf_counter() - h0) * 1e3 / R)
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        avg[n] = float(np.mean([a.elapsed_time(b) for a, b in pairs])) / R
        host_launch_ms[n] = float(np.mean(hs))
    del pre_sets, dec_sets, states

    # The same prefill replayed as one HIP graph (one launch for three
    # kernels), timed after an eviction in the same way; reported beside.
    G_pre = capture(g_dt, g_select, g_attn)
    gpairs = []
    for _ in range(args.steps):
        evict()
        a, b = ev(), ev()
        a.record()
        G_pre.replay()
        b.record()
        gpairs.append((a, b))
    torch.cuda.synchronize()
    ms_pre_graph = float(np.mean([a.elapsed_time(b) for a, b in gpairs]))

    flops = kept_flops(wl_p.B, wl_p.Hq, wl_p.S, wl_p.d, wl_p.w)
    value = flops / (ms_pre * 1e-3) / 1e12
    dbytes = decode_bytes(wl_d.B, wl_d.Hq, wl_d.Hkv, wl_d.d, wl_d.w, dec["cache_lens"])
    dec_gbs = dbytes / (avg["decode"] * 1e-3) / 1e9
    attn_tflops = flops / (avg["attn_fwd"] * 1e-3) / 1e12
    sbytes = decode_state_bytes_moved(wl_d.B, wl_d.Hq, wl_d.Hkv, wl_d.d, wl_d.w, pos.cpu().numpy())
    step_gbs = sbytes / (avg["decode_step"] * 1e-3) / 1e9
    pbytes = prologue_bytes(wl_p.B, wl_p.S, wl_p.Hq, wl_p.Hkv, wl_p.d)
    pro_gbs = pbytes / (avg["prologue"] * 1e-3) / 1e9
    ms_bwd = avg["attn_bwd"] + avg["dt_bwd"]
    bwd_tflops = 2.5 * flops / (ms_bwd * 1e-3) / 1e12

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
            "ms_per_launch": round(avg["attn_fwd"], 5), "flop_per_launch": flops,
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 5),
            "traffic": (ATTN_TRAFFIC["bytes"]
                        if ATTN_TRAFFIC["sources_sha256"] == sources_sha256(ATTN_SOURCES) else None),
        },
        "decode": {
            "value": round(dec_gbs, 2), "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
            "frac": round(dec_gbs / PEAK_HBM_GBS, 5),
        },
        "decode_incremental": {
            "value": round(step_gbs, 2), "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
            "frac": round(step_gbs / PEAK_HBM_GBS, 5), "bytes": sbytes, "ms": round(avg["decode_step"], 5),
            "tokens_per_s": round(wl_d.B / (avg["decode_step"] * 1e-3), 1),
            "note": "dma_decode_step: kept set carried across steps, the kept K/V rows stored compactly",
        },
        "prologue": {
            "value": round(pro_gbs, 2), "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
            "frac": round(pro_gbs / PEAK_HBM_GBS, 5), "bytes": pbytes, "ms": round(avg["prologue"], 5),
            "note": "dma_prologue on the prefill workload, in place: Q/K RMSNorm + rotary, then dt",
        },
        "backward": {
            "value": round(bwd_tflops, 3), "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
            "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 5), "flops": 2.5 * flops, "ms": round(ms_bwd, 5),
            "note": "dma_attn_bwd + dma_dt_bwd on the prefill workload; kept-key flops of the five products "
                    "(scores, dp, dq, dk, dv) = 2.5x the forward's",
        },
        "ms_prefill": round(ms_pre, 5),
        "ms_decode_step": round(ms_dec, 5),
        "step_ms_percentiles": {
            n: {q: round(float(np.percentile(v, int(q[1:]))), 5) for q in ("p10", "p50", "p90")}
            for n, v in (("prefill", pre_each), ("decode", dec_each))},
        "kernel_ms_avg": {n: round(v, 5) for n, v in avg.items()},
        "ms_prefill_as_one_graph": round(ms_pre_graph, 5),
        "host_enqueue_ms_per_step": round(float(np.mean(host_ms)), 4),
        "host_ms_per_launch": {n: round(v, 5) for n, v in host_launch_ms.items()},
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
    }
    line["window_variant"] = window_breakdown(dma, dev, evict)
    line["cdmoe"] = cdmoe_breakdown(dma, dev, evict)
    if args.other_configs:
        line["other_configs"] = {n: prefill_breakdown(dma, n, dev, evict) for n in ("long", "padded")}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pre, wl_p)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

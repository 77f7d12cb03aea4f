"""Benchmark of the DMA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-variants]
    python bench.py --copy-calibration     (a plain 256 MiB copy, for counter scaling)
    python bench.py --attn-only NAME       (a few attention launches of one prefill workload)

One step = the whole hot path over one batch of synthetic input:
  prefill  B=2 Hq=16 Hkv=4 S=32768 d=128 w=2048 bf16, right-padded lengths
           ~ U[16384, 32768] (dma_dt -> dma_select -> dma_attn_fwd)
  decode   B=64 Hq=8 Hkv=2 d=128 w=2048, 16384 cached positions
           (dma_dt appends the new token's dt, then dma_decode)
A 512 MiB read before each half evicts the inputs from the caches (with
clean lines, so no write-back traffic lands on the timed calls); the
evictions are outside the timed kernels.

Printed: ONE JSON line.  value = prefill kept-key TFLOP/s of the padded
workload (kept (query, key) pairs x 4*d flop over the GPU time of the three
prefill calls, launched back to back); the decode GB/s (algorithmic bytes
over dma_decode's GPU time) rides along under "decode".  The long
(B1 Hq16 Hkv8 S8192 d128 w2048) and c2 (B4 Hq8 Hkv4 S2048 d64 w512) prefill
workloads are timed per call under "prefill_configs".  ms_per_step = prefill
+ decode GPU time of one step.  Times come from HIP events recorded between
the calls on the stream the kernels run on (torch's current stream, which
the binding launches on).
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

GPU_WARM_S = 0.25   # untimed steps that bring the GPU's clocks up before the W warm-up steps

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak

# HBM bytes per launch of the padded workload's attention kernel, from two
# rocprofv3 counter runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch), each scaled by copy_bytes / counter reading of a plain copy of
# known size (--copy-calibration); the runs and their readings are in
# profiles/.  The figure holds only for the attention source it was measured
# on: when the hash of those files differs, traffic is reported as null.
ATTN_TRAFFIC = {"bytes": 764028560,
                "sources_sha256": "e8dfaa6b23cacf0d2b3eacf113e4081132fc6af9b47e2c2700fdc34400d03b8e"}
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



def host_cpu_info():
    """CPU model, sockets and core counts of this host."""
    model, phys, ids = "", set(), {}
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                key = ln.split(":", 1)[0].strip()
                if key == "model name" and not model:
                    model = ln.split(":", 1)[1].strip()
                elif key == "physical id":
                    phys.add(ln.split(":", 1)[1].strip())
                elif key in ("cpu family", "model", "stepping") and key not in ids:
                    ids[key] = ln.split(":", 1)[1].strip()
    except OSError:
        pass
    if ids:  # a virtualised host may name only the product line
        model += " (family %s, model %s, stepping %s)" % (ids.get("cpu family", "?"), ids.get("model", "?"),
                                                         ids.get("stepping", "?"))
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "sockets": max(1, len(phys)), "nproc": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(inp, wl, rows_per_unit=1024, reps=3):
    """The oracle (plain C, fp64, OpenMP over rows) timed on the host on a
    stratified sample of the prefill workload: dt over every token, then the
    selection and the attention of rows_per_unit rows per (batch, kv head),
    evenly spaced over [0, L_b) (so the rows before and after the first w
    keys are represented as in the full workload).  Each stage runs once to
    warm up, then reps times; the median is taken.  value = kept-key flops of
    the sampled rows / (select + attention time of the sample + the dt time
    prorated to the sampled share of the rows)."""
    import oracle
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or (os.cpu_count() or 1)
    L = inp["seqlens"] if inp["seqlens"] is not None else np.full(wl.B, wl.S, np.int32)
    rows = sorted({(b, g, int(i)) for b in range(wl.B) for g in range(wl.Hkv)
                   for i in np.linspace(0, int(L[b]) - 1, rows_per_unit).round()})
    rows = np.array(rows, dtype=np.int32)
    G = wl.Hq // wl.Hkv
    sample_flops = int(sum(4 * wl.d * G * min(int(i) + 1, wl.w) for _, _, i in rows))
    total_rows = int(sum(int(x) for x in L)) * wl.Hkv
    total_flops = kept_flops(wl.B, wl.Hq, wl.S, wl.d, wl.w, inp["seqlens"])

    def timed(fn):
        fn()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            r = fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)), r

    t_dt, dt64 = timed(lambda: oracle.dt(inp["V"], inp["W"], inp["bias"], inp["A"]))
    dt32 = dt64.astype(np.float32)
    t_sel, _ = timed(lambda: oracle.select(dt32, wl.w, inp["seqlens"], rows=rows))
    t_attn, _ = timed(lambda: oracle.attn(inp["Q"], inp["K"], inp["V"], dt32, wl.w, inp["seqlens"], rows=rows))
    share = len(rows) / total_rows
    t_sample = t_sel + t_attn + t_dt * share
    return {"value": sample_flops / t_sample / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {total_rows} (batch, kv head, row) rows of the padded prefill, "
                      f"{rows_per_unit} per (batch, kv head) evenly spaced over its valid rows, each with its "
                      f"{G} query heads; dt over all tokens prorated to that share; fp64; median of {reps} "
                      f"runs after one warm-up",
            "sample_kept_flops": sample_flops,
            "stage_s": {"dt_all_tokens": round(t_dt, 4), "select_sample": round(t_sel, 4),
                        "attn_sample": round(t_attn, 4)},
            "est_full_prefill_s": round(t_dt + t_sel / share + t_attn * total_flops / sample_flops, 2),
            "host": {**host_cpu_info(), "omp_threads": threads}}


def per_launch_ms(calls, evict, R, rounds):
    """Average GPU time per launch of each call: after untimed launches that
    bring the clocks up, an eviction, then R back-to-back launches between two
    events, `rounds` times."""
    res, host = {}, {}
    for n, f in calls:
        f()                         # the first launch of a kernel loads its code
        torch.cuda.synchronize()
        # untimed launches for GPU_WARM_S / 5, so that a call timed after a
        # quiet or memory-bound stretch runs at the clocks of sustained work
        t_w, k = time.perf_counter(), 0
        while time.perf_counter() - t_w < GPU_WARM_S / 5:
            f()
            k += 1
            if k % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        pairs, hs = [], []
        for _ in range(rounds):
            evict()
            evict()                 # keeps the GPU busy while the host enqueues the R launches
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            h0 = time.perf_counter()
            for _ in range(R):
                f()
            hs.append((time.perf_counter() - h0) * 1e3 / R)
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        res[n] = float(np.mean([a.elapsed_time(b) for a, b in pairs])) / R
        host[n] = float(np.mean(hs))
    return res, host


class Prefill:
    """One prefill workload on the device, with rotating copies of its
    inputs (enough that the data read between two launches of a call exceeds
    the 256 MB last-level cache, so every launch reads from HBM)."""

    def __init__(self, dma, name, dev, inp=None):
        self.dma, self.name = dma, name
        self.wl = wl = si.WORKLOADS[name]
        self.inp = inp = si.make_inputs(wl) if inp is None else inp
        self.Q, self.K, self.V = to_dev(inp["Q"], dev), to_dev(inp["K"], dev), to_dev(inp["V"], dev)
        self.W, self.A, self.bias = to_dev(inp["W"], dev), to_dev(inp["A"], dev), to_dev(inp["bias"], dev)
        self.seq = None if inp["seqlens"] is None else to_dev(inp["seqlens"], dev)
        self.dt = torch.empty((wl.B, wl.Hkv, wl.S), dtype=torch.float32, device=dev)
        self.tau = torch.empty_like(self.dt)
        self.tie = torch.empty(self.dt.shape, dtype=torch.int32, device=dev)
        self.O = torch.empty_like(self.Q)
        dma.dt(self.V, self.W, self.A, self.bias, out=self.dt)
        dma.select(self.dt, wl.w, self.seq, tau=self.tau, tie=self.tie)
        self.flops = kept_flops(wl.B, wl.Hq, wl.S, wl.d, wl.w, inp["seqlens"])
        self.sets, self.rot, self.ncopies = None, 0, 1

    def make_sets(self, min_bytes=300 * 2**20):
        first = (self.Q, self.K, self.V, self.dt, self.tau, self.tie)
        set_bytes = sum(t.numel() * t.element_size() for t in first)
        n = 1 + -(-min_bytes // set_bytes)
        self.sets = [first] + [tuple(t.clone() for t in first) for _ in range(n - 1)]
        self.ncopies = n

    def drop_sets(self):
        self.sets = None

    def nxt(self):
        self.rot += 1
        return self.sets[self.rot % len(self.sets)]

    # the three calls of the path on the resident inputs (no rotation)
    def g_dt(self):
        self.dma.dt(self.V, self.W, self.A, self.bias, out=self.dt)

    def g_select(self):
        self.dma.select(self.dt, self.wl.w, self.seq, tau=self.tau, tie=self.tie)

    def g_attn(self):
        self.dma.attn_fwd(self.Q, self.K, self.V, self.dt, self.tau, self.tie, self.wl.w, self.seq, out=self.O)

    # the same calls, each on the next copy of the inputs
    def c_dt(self):
        s_ = self.nxt()
        self.dma.dt(s_[2], self.W, self.A, self.bias, out=s_[3])

    def c_select(self):
        s_ = self.nxt()
        self.dma.select(s_[3], self.wl.w, self.seq, tau=s_[4], tie=s_[5])

    def c_attn(self):
        s_ = self.nxt()
        self.dma.attn_fwd(*s_, self.wl.w, self.seq, out=self.O)

    def summary(self, ms):
        tot = ms["dt"] + ms["select"] + ms["attn_fwd"]
        wl = self.wl
        att = self.flops / (ms["attn_fwd"] * 1e-3) / 1e12
        return {"workload": workload_name(wl), "ms": {k: round(v, 5) for k, v in ms.items()},
                "kept_flops": self.flops, "input_copies": self.ncopies,
                "tflops_prefill": round(self.flops / (tot * 1e-3) / 1e12, 2), "tflops_attn": round(att, 2),
                "attn_frac_of_peak": round(att / PEAK_BF16_TFLOPS, 4),
                "select_share_of_prefill": round(ms["select"] / tot, 4)}


def workload_name(wl):
    pad = f", right-padded lengths ~U[{wl.pad_lo},{wl.pad_hi}]" if wl.pad_hi else ""
    return f"prefill B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} S{wl.S} d{wl.d} w{wl.w} {wl.dtype}{pad}"


def attn_only(name, launches):
    """A few attention launches of one prefill workload (for counter runs):
    the inputs are built, dt and the thresholds computed once, then
    `launches` launches of dma_attn_fwd on rotating input copies."""
    import doge_dynamic_mask_amd as dma
    dma.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    P = Prefill(dma, name, dev)
    P.make_sets()
    for _ in range(launches):
        P.c_attn()
    torch.cuda.synchronize()
    print(json.dumps({"attn_only": name, "launches": launches, "kept_flops": P.flops}), flush=True)


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
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the sliding-window and CDMoE measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain copies of known size (counter calibration)")
    ap.add_argument("--attn-only", default=None, help="only run attention launches of this prefill workload")
    ap.add_argument("--launches", type=int, default=5)
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the DMA hot path here has no cross-GPU step "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.attn_only:
        attn_only(args.attn_only, args.launches)
        return

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    import doge_dynamic_mask_amd as dma
    dma.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    progress("inputs: padded prefill")
    P5 = Prefill(dma, "padded", dev)
    wl_p = P5.wl
    wl_d = si.WORKLOADS["decode"]
    progress("inputs: decode")
    dec = si.make_inputs(wl_d)
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

    def g_dt_append():
        dma.dt(v_new, Wd, Ad, biasd, out=dt_cache, out_pos=pos)

    def g_decode():
        dma.decode(q, Kc, Vc, dt_cache, lens, wl_d.w, out=out, workspace=ws)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # One step: evict, the three prefill calls back to back, evict, the two
    # decode calls.
    PRE = (P5.g_dt, P5.g_select, P5.g_attn)
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

    # The GPU raises its clocks over the first tens of milliseconds of
    # sustained work after an idle spell such as the host-side input
    # generation above (measured: the padded prefill takes 1.2 ms in the first
    # steps, 1.10 ms on average over steps 5-25 and 0.99 ms from about the
    # 35th step on).  So untimed steps of the same work run for
    # GPU_WARM_S first; then the W warm-up steps and the K timed ones.
    progress(f"gpu warm-up: untimed steps for {GPU_WARM_S} s")
    t_w, n_w = time.perf_counter(), 0
    while n_w < 20 or time.perf_counter() - t_w < GPU_WARM_S:
        step()
        n_w += 1
        if n_w % 20 == 0:
            torch.cuda.synchronize()    # the host stays at most 20 steps ahead
    torch.cuda.synchronize()
    gpu_warm = {"s": round(time.perf_counter() - t_w, 3), "steps": n_w}
    progress(f"steps: {args.warmup} warm-up, {args.steps} timed")
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

    # Per-launch times of every call (rotating input copies, see Prefill).
    progress("per-launch: padded prefill")
    P5.make_sets()
    avg5, host5 = per_launch_ms((("dt", P5.c_dt), ("select", P5.c_select), ("attn_fwd", P5.c_attn)),
                                evict, R=6, rounds=4)
    # the prologue upstream of dt (Q/K RMSNorm + rotary, then dt), in place on
    # the rotating copies; timed after attn_fwd, whose inputs it rewrites
    wq5, wk5 = (to_dev(x, dev) for x in si.make_norm_weights(wl_p.d, wl_p.dtype, wl_p.seed + 7))

    def c_prologue5():
        q_, k_, v_, d, _, _ = P5.nxt()
        dma.prologue(q_, k_, v_, wq5, wk5, P5.W, P5.A, P5.bias, Q_out=q_, K_out=k_, dt_out=d)
    pro5, _ = per_launch_ms((("prologue", c_prologue5),), evict, R=6, rounds=3)
    P5.drop_sets()

    progress("per-launch: decode")
    NDEC = 4     # decode caches (~134 MB of kept rows each)
    dec_sets = [(Kc, Vc, dt_cache)] + [tuple(t.clone() for t in (Kc, Vc, dt_cache)) for _ in range(NDEC - 1)]
    rot = [0]

    def nxt_dec():
        rot[0] += 1
        return dec_sets[rot[0] % NDEC]

    def c_dt_append():
        dma.dt(v_new, Wd, Ad, biasd, out=nxt_dec()[2], out_pos=pos)

    def c_decode():
        kc, vc, dc = nxt_dec()
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

    avg_d, host_d = per_launch_ms((("dt_append", c_dt_append), ("decode", c_decode),
                                   ("decode_step", c_decode_step)), evict, R=12, rounds=5)
    del dec_sets, states

    progress("per-launch: long and c2 prefill, backward, prologue")
    P3 = Prefill(dma, "long", dev)
    P3.make_sets()
    avg3, _ = per_launch_ms((("dt", P3.c_dt), ("select", P3.c_select), ("attn_fwd", P3.c_attn)),
                            evict, R=8, rounds=4)
    P3.drop_sets()
    P2 = Prefill(dma, "c2", dev)
    P2.make_sets()
    wl2 = P2.wl
    wq, wk = (to_dev(x, dev) for x in si.make_norm_weights(wl2.d, wl2.dtype, wl2.seed + 7))

    def c_qk_norm_rope():
        q_, k_, _, _, _, _ = P2.nxt()
        dma.qk_norm_rope(q_, k_, wq, wk, Q_out=q_, K_out=k_)

    def c_prologue():
        q_, k_, v_, d, _, _ = P2.nxt()
        dma.prologue(q_, k_, v_, wq, wk, P2.W, P2.A, P2.bias, Q_out=q_, K_out=k_, dt_out=d)

    dO = torch.randn_like(P2.Q)
    ws_b = torch.empty(dma.attn_bwd_workspace_bytes(wl2.B, wl2.S, wl2.Hq, wl2.Hkv, wl2.d, wl2.w),
                       dtype=torch.uint8, device=dev)
    ws_db = torch.empty(dma.dt_bwd_workspace_bytes(wl2.B, wl2.S, wl2.Hkv, wl2.d), dtype=torch.uint8, device=dev)
    g_out = (torch.empty_like(P2.Q), torch.empty_like(P2.K), torch.empty_like(P2.V), torch.empty_like(P2.dt))

    def c_attn_bwd():
        q_, k_, v_, d, ta, ti = P2.nxt()
        dma.attn_bwd(q_, k_, v_, d, ta, ti, wl2.w, dO, workspace=ws_b, out=g_out)

    def c_dt_bwd():
        _, _, v_, _, _, _ = P2.nxt()
        dma.dt_bwd(v_, P2.W, P2.A, g_out[3], P2.bias, dV=g_out[2], workspace=ws_db)

    avg2, host2 = per_launch_ms((("dt", P2.c_dt), ("select", P2.c_select), ("attn_fwd", P2.c_attn),
                                 ("attn_bwd", c_attn_bwd), ("dt_bwd", c_dt_bwd),
                                 ("qk_norm_rope", c_qk_norm_rope), ("prologue", c_prologue)),
                                evict, R=12, rounds=5)
    P2.drop_sets()

    # The padded prefill replayed as one HIP graph (one launch for three
    # kernels), timed after an eviction in the same way; reported beside.
    for f in PRE:
        f()
    torch.cuda.synchronize()
    G_pre = torch.cuda.CUDAGraph()
    with torch.cuda.graph(G_pre):
        for f in PRE:
            f()
    torch.cuda.synchronize()
    gpairs = []
    for _ in range(max(3, args.steps // 2)):
        evict()
        a, b = ev(), ev()
        a.record()
        G_pre.replay()
        b.record()
        gpairs.append((a, b))
    torch.cuda.synchronize()
    ms_pre_graph = float(np.mean([a.elapsed_time(b) for a, b in gpairs]))

    flops = P5.flops
    value = flops / (ms_pre * 1e-3) / 1e12
    dbytes = decode_bytes(wl_d.B, wl_d.Hq, wl_d.Hkv, wl_d.d, wl_d.w, dec["cache_lens"])
    dec_gbs = dbytes / (avg_d["decode"] * 1e-3) / 1e9
    attn_tflops = flops / (avg5["attn_fwd"] * 1e-3) / 1e12
    sbytes = decode_state_bytes_moved(wl_d.B, wl_d.Hq, wl_d.Hkv, wl_d.d, wl_d.w, pos.cpu().numpy())
    step_gbs = sbytes / (avg_d["decode_step"] * 1e-3) / 1e9
    pbytes2 = prologue_bytes(wl2.B, wl2.S, wl2.Hq, wl2.Hkv, wl2.d)
    pbytes5 = prologue_bytes(wl_p.B, wl_p.S, wl_p.Hq, wl_p.Hkv, wl_p.d)
    ms_bwd = avg2["attn_bwd"] + avg2["dt_bwd"]
    bwd_tflops = 2.5 * P2.flops / (ms_bwd * 1e-3) / 1e12
    traffic_ok = ATTN_TRAFFIC["bytes"] is not None and \
        ATTN_TRAFFIC["sources_sha256"] == sources_sha256(ATTN_SOURCES)

    line = {
        "metric": "DMA prefill kept-key TFLOP/s + decode GB/s, % of MI355X roofline",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "gpu_warmup": gpu_warm,
        "ms_per_step": round(ms_pre + ms_dec, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, N(0,0.02) dt_proj, A~U(-2,2), lengths ~U[16384,32768])",
        "config": {
            "workload": workload_name(wl_p) + " (dt+select+attn) + decode B64 L16384 Hq8 Hkv2 d128 w2048 "
                        "(dt append + decode)",
            "prefill_kept_flops": flops,
            "prefill_lengths": [int(x) for x in P5.inp["seqlens"]],
            "decode_bytes": dbytes,
        },
        "roofline": {
            "bound": "mfma", "kernel": "dma_attn_fwd (attn_bf16_kernel<128>) on the padded workload",
            "achieved": round(attn_tflops, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 5),
            "traffic": ATTN_TRAFFIC["bytes"] if traffic_ok else None,
            "ms_per_launch": round(avg5["attn_fwd"], 5), "flop_per_launch": flops,
        },
        "prefill_configs": {"padded": P5.summary(avg5), "long": P3.summary(avg3),
                            "c2": P2.summary({k: avg2[k] for k in ("dt", "select", "attn_fwd")})},
        "decode": {
            "value": round(dec_gbs, 2), "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
            "frac": round(dec_gbs / PEAK_HBM_GBS, 5), "bytes": dbytes, "ms": round(avg_d["decode"], 5),
        },
        "decode_incremental": {
            "value": round(step_gbs, 2), "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
            "frac": round(step_gbs / PEAK_HBM_GBS, 5), "bytes": sbytes, "ms": round(avg_d["decode_step"], 5),
            "tokens_per_s": round(wl_d.B / (avg_d["decode_step"] * 1e-3), 1),
            "note": "dma_decode_step: kept set carried across steps, the kept K/V rows stored compactly",
        },
        "prologue": {
            "padded": {"value": round(pbytes5 / (pro5["prologue"] * 1e-3) / 1e9, 2), "unit": "GB/s",
                       "frac": round(pbytes5 / (pro5["prologue"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
                       "bytes": pbytes5, "ms": round(pro5["prologue"], 5)},
            "c2": {"value": round(pbytes2 / (avg2["prologue"] * 1e-3) / 1e9, 2), "unit": "GB/s",
                   "frac": round(pbytes2 / (avg2["prologue"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
                   "bytes": pbytes2, "ms": round(avg2["prologue"], 5)},
            "bound": "hbm", "peak": PEAK_HBM_GBS,
            "note": "dma_prologue in place: Q/K RMSNorm + rotary, then dt",
        },
        "backward": {
            "value": round(bwd_tflops, 3), "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
            "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 5), "flops": 2.5 * P2.flops, "ms": round(ms_bwd, 5),
            "note": "dma_attn_bwd + dma_dt_bwd on the c2 workload; kept-key flops of the five products "
                    "(scores, dp, dq, dk, dv) = 2.5x the forward's",
        },
        "ms_prefill": round(ms_pre, 5),
        "ms_decode_step": round(ms_dec, 5),
        "step_ms_percentiles": {
            n: {q_: round(float(np.percentile(v, int(q_[1:]))), 5) for q_ in ("p10", "p50", "p90")}
            for n, v in (("prefill", pre_each), ("decode", dec_each))},
        "kernel_ms_avg": {"padded": {k: round(v, 5) for k, v in avg5.items()},
                          "decode": {k: round(v, 5) for k, v in avg_d.items()},
                          "c2": {k: round(v, 5) for k, v in avg2.items()}},
        "ms_prefill_as_one_graph": round(ms_pre_graph, 5),
        "host_enqueue_ms_per_step": round(float(np.mean(host_ms)), 4),
        "host_ms_per_launch": {**{f"padded_{k}": round(v, 5) for k, v in host5.items()},
                               **{f"decode_{k}": round(v, 5) for k, v in host_d.items()},
                               **{f"c2_{k}": round(v, 5) for k, v in host2.items()}},
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
    }
    del P3, P2
    if not args.no_variants:
        progress("variants: sliding window, CDMoE")
        line["window_variant"] = window_breakdown(dma, dev, evict)
        line["cdmoe"] = cdmoe_breakdown(dma, dev, evict)
    if not args.no_cpu_baseline:
        progress("cpu baseline: the oracle on a row sample of the padded prefill")
        line["cpu_baseline"] = cpu_baseline(P5.inp, wl_p)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

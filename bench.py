#!/usr/bin/env python3
"""Benchmark of the paged, heterogeneous-batch LoRA delta on one MI355X.

One step is one pass of the hot path over one batch: the shrink kernel
(v = x A from the A^T pages) and the expand kernel (y += s v B from the B
pages) for every token of the batch, with the batch's segment metadata, x, y
and the adapter pages already resident in HBM.  Before every step a 1 GiB
device copy evicts the 256 MB last-level cache, so each step reads its pages
from HBM as a serving iteration would after the rest of the model ran; the
copy sits outside the HIP events that time the step.  Host segment building
and the metadata upload (PCIe) are timed on their own and reported beside the
step, never inside ``value``.

Prints one JSON line: tokens/s, per-kernel times, the roofline of the dominant
kernel against MI355X's 8 TB/s HBM, and the fp64 CPU oracle's rate on the
host cores (``cpu_baseline``).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak
METRIC = "LoRA-delta tokens/s + achieved HBM GB/s (decode) / MFMA util (prefill)"
WORKLOAD_NOTES = {
    "tiny": "H 256->256 fp32, 4 adapters r{4,8,4,8}, 16 tokens uniform ids, 128-page shuffled pool",
    "decode7b": "Llama-7B shape 4096->4096 fp16, 1000 adapters r in {8,16,32,64}, 256 decode tokens "
                "with Zipf(1.1) adapter ids, A/B pages scattered among 60% KV pages",
    "prefill7b": "Llama-7B shape 4096->4096 fp16, 32 requests of 64..512 tokens, one of 100 adapters "
                 "each, shuffled pool at 50% KV",
    "mixed13b": "Llama-13B 5120->5120 fp16, q,k,v,o projections, 2000 adapters, 8x256 prefill + "
                "384 decode tokens, uniform ids",
    "mlp70b": "8192->28672 fp16, two page classes, 5000 adapters r in {16,32,64,128}, 512 decode "
              "tokens Zipf(1.0), pool 80% KV",
}


def workload(name, seed, rank_pad=0):
    """The named synthetic batch; with rank_pad > 0, the same batch with every
    adapter's rank rounded up to a multiple of rank_pad (at most 256), as a
    layout that pads ranks to uniform tiles would store it (token ids, x and y
    come from their own random streams and stay as they were)."""
    from synth import CONFIGS, generate

    w = generate(CONFIGS[name], seed)
    if rank_pad:
        padded = tuple(min(256, -(-int(r) // rank_pad) * rank_pad) for r in w.ranks)
        w = generate(dataclasses.replace(CONFIGS[name], fixed_ranks=padded), seed)
    return w


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def load_traffic(config, dominant, kind="fused"):
    """(HBM bytes per launch, rocprofv3 kernel-trace average us) from the committed
    rocprofv3 summary of this workload, if it was taken of the current kernels.
    kind "forward": the base-plus-delta launches of one call, summed."""
    name = f"traffic_{config}.json" if kind == "fused" else f"traffic_{kind}_{config}.json"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        t = json.load(f)
    from rank_gemm_page_amd.profiling import kernel_source_hash
    if t.get("kernel_source_hash") != kernel_source_hash(kind):
        return None, None
    ks = [v for k, v in t.get("kernels", {}).items() if k == dominant or (kind != "fused" and k.startswith(dominant))]
    if not ks:
        return None, None
    avg = [k.get("trace_avg_us") for k in ks]
    return (sum(k["fetch_bytes"] + k["write_bytes"] for k in ks),
            sum(avg) if all(a is not None for a in avg) else None)


def load_mfma_util(config):
    """Matrix-core busy share and issued fp16 MFMA flops of the fused kernel
    from the committed rocprofv3 counter run of this workload, if it was taken
    of the current kernels."""
    path = os.path.join(ROOT, "profiles", f"mfma_{config}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    from rank_gemm_page_amd.profiling import kernel_source_hash
    if t.get("kernel_source_hash") != kernel_source_hash("fused"):
        return None
    return {"mfma_util_percent": t["mfma_util_percent"],
            "mfma_flops_f16_per_launch": t["mfma_flops_f16_per_launch"],
            "source": f"profiles/mfma_{config}.json ({t['counters']})"}


def cpu_baseline(w, budget_s=10.0, one_thread=True):
    """The fp64 oracle on the host cores over a bounded sample of the batch."""
    import numpy as np

    from oracle import build_from_workload, workload_delta
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = None
    st = build_from_workload(w)
    n_proj = w.spec.n_proj
    t = time.perf_counter()
    workload_delta(st, w, proj=0, tokens=[0])
    per_tok = max((time.perf_counter() - t) * n_proj, 1e-5)
    # One pass = the sampled tokens through every projection of the step; passes
    # repeat until about budget_s of CPU work is done.
    n = int(min(w.T, max(1, budget_s / per_tok)))
    toks = np.linspace(0, w.T - 1, n).astype(int).tolist()

    def rate(budget):
        passes, elapsed = 0, 0.0
        while elapsed < budget or passes < 2:
            t = time.perf_counter()
            for p in range(n_proj):
                workload_delta(st, w, proj=p, tokens=toks)
            elapsed += time.perf_counter() - t
            passes += 1
        return passes, elapsed

    passes, elapsed = rate(budget_s)
    out = {"value": passes * n / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} of {w.T} tokens of the same batch through all {n_proj} projection(s), "
                     f"{passes} passes in {elapsed:.1f} s, fp64 NumPy, page-table walk per token",
           "host_cpu_count": os.cpu_count()}
    # the same sample with the BLAS pool held to one thread, a shorter run
    if not one_thread:
        return out
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            p1, e1 = rate(budget_s / 3)
        out["value_1_thread"] = p1 * n / e1
    except Exception:
        out["value_1_thread"] = None
    return out


class BmmPath:
    """The ablation baseline of the summary page ("Results & figures", Figure 5
    narrative: the custom kernels replaced by a slower BMM path), read as the
    plain batched-matmul LoRA: the batch's adapters as dense tensors padded
    with zeros to the largest rank (built once per batch from the pool pages,
    not timed), then per step a per-token gather of those tensors, two torch
    bmm calls (x A, then (x A) B) and y[t] = y[t] + s_a d[t] in fp32 with one
    rounding.  torch only, as a comparison; it is not the product path."""

    def __init__(self, dw, proj=0):
        import numpy as np
        import torch

        from rank_gemm_page_amd import slora as S
        w, info, dev = dw.w, dw.info, dw.device
        ex = S.slora_segments_export(dw.seg)
        n_seg, sum_r = info["n_segments"], info["sum_rank"]
        ranks = ex["seg_rank"]
        rmax = int(ranks.max()) if n_seg else 1
        b_cls = 1 if w.spec.two_classes else 0
        self.A = torch.zeros(max(n_seg, 1), w.spec.h_in, rmax, dtype=dw.tdtype, device=dev)
        self.B = torch.zeros(max(n_seg, 1), rmax, w.spec.h_out, dtype=dw.tdtype, device=dev)
        sidx = np.full(w.T, -1, np.int64)
        for g in range(n_seg):
            r, o = int(ranks[g]), proj * sum_r + int(ex["seg_page_off"][g])
            ida = torch.from_numpy(ex["a_pages"][o:o + r].astype(np.int64)).to(dev)
            idb = torch.from_numpy(ex["b_pages"][o:o + r].astype(np.int64)).to(dev)
            self.A[g, :, :r] = dw.pages[0].index_select(0, ida).t()
            self.B[g, :r, :] = dw.pages[b_cls].index_select(0, idb)
            sidx[ex["perm"][ex["seg_start"][g]:ex["seg_start"][g + 1]]] = g
        tok = np.nonzero(sidx >= 0)[0]
        self.tok = torch.from_numpy(tok).to(dev)
        self.sidx = torch.from_numpy(sidx[tok]).to(dev)
        self.scale = torch.from_numpy(ex["seg_scale"][sidx[tok]].astype(np.float32)).to(dev)[:, None]
        self.rmax = rmax

    def step(self, x, y):
        import torch
        if self.tok.numel() == 0:
            return
        a_t = self.A.index_select(0, self.sidx)                    # [n, h_in, rmax]
        b_t = self.B.index_select(0, self.sidx)                    # [n, rmax, h_out]
        v = torch.bmm(x.index_select(0, self.tok).unsqueeze(1), a_t)
        d = torch.bmm(v, b_t).squeeze(1)
        y[self.tok] = (y.index_select(0, self.tok).float() + self.scale * d.float()).to(y.dtype)


def measure_bmm_path(dw, w, steps, flush, stream, paged_ms):
    import torch
    paths = [BmmPath(dw, p) for p in range(w.spec.n_proj)]

    def run():
        for p, bp in enumerate(paths):
            bp.step(dw.x[w.spec.proj_x[p]], dw.y[p])

    for _ in range(2):
        flush()
        run()
    ts = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flush()
        a.record(stream)
        run()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ms = statistics.fmean(ts)
    tokens = int(paths[0].tok.numel())
    e = 2 if w.spec.dtype == "f16" else 4
    gathered = sum(int(bp.tok.numel()) * bp.rmax * (w.spec.h_in + w.spec.h_out) * e for bp in paths)
    return {"ms_per_step": round(ms, 5), "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s",
            "paged_speedup": round(ms / paged_ms, 2), "padded_rank": paths[0].rmax,
            "gathered_weight_bytes": gathered,
            "method": "per-token gather of zero-padded dense adapters + 2 torch.bmm + fp32 scaled add; "
                      "HIP events, cache flushed before each step"}


def measure_base_gemm(dw, w, steps, flush, stream, paged_ms):
    """Context for the summary page's claim that the LoRA work is cheap next to
    the base xW ("The mechanism", separate base and delta): the same step's
    base products x W (one dense h_in x h_out fp16/fp32 weight per projection,
    random, torch.mm on hipBLASLt) timed like the delta, flush included."""
    import torch
    spec = w.spec
    wts = [torch.randn(spec.h_in, spec.h_out, device=dw.device).to(dw.tdtype) * 0.02
           for _ in range(spec.n_proj)]
    outs = [torch.empty(w.T, spec.h_out, dtype=dw.tdtype, device=dw.device) for _ in range(spec.n_proj)]

    def run():
        for p in range(spec.n_proj):
            torch.mm(dw.x[spec.proj_x[p]], wts[p], out=outs[p])

    for _ in range(3):
        flush()
        run()
    ts = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flush()
        a.record(stream)
        run()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ms = statistics.fmean(ts)
    flops = 2.0 * w.T * spec.h_in * spec.h_out * spec.n_proj
    return {"ms_per_step": round(ms, 5), "TFLOPs": round(flops / (ms * 1e-3) / 1e12, 1),
            "delta_over_base": round(paged_ms / ms, 4),
            "y_round_trip_bytes": 2 * w.T * spec.h_out * spec.n_proj * (2 if spec.dtype == "f16" else 4),
            "method": "torch.mm(x, W) per projection, random W, HIP events, cache flushed before each step"}


def measure_prefetch(dw, w, m, steps, flush, step, stream):
    """Walkthrough step 2 of the summary page: the next batch's adapters are
    fetched into the pool while the current batch computes.  m adapters the
    batch does not reference are evicted, then fetched again from pinned host
    images on a second stream, first alone and then while the step's delta
    runs; after every step they are evicted again.  One
    slora_load_adapters_async call per step queues all m image copies and one
    scatter launch."""
    import numpy as np
    import torch

    from rank_gemm_page_amd import slora as S
    cand = [a for a in range(w.spec.n_adapters) if not w.referenced[a]][:m]
    images = {a: dw.pack(a) for a in cand}
    for a in cand:
        S.slora_unload_adapter(dw.pool, a)
    side = torch.cuda.Stream()
    nbytes = sum(int(w.spec.n_proj * w.ranks[a] * (w.spec.h_in + w.spec.h_out)
                     * (2 if w.spec.dtype == "f16" else 4)) for a in cand)

    def fetch_round(with_delta):
        t0, td, tl = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        flush()
        t0.record(stream)
        side.wait_event(t0)
        if with_delta:
            step()
            td.record(stream)
        h = time.perf_counter()
        dw.load_async(cand, side, images=[images[a] for a in cand])
        host_s = time.perf_counter() - h
        tl.record(side)
        torch.cuda.synchronize()
        dw.images.clear()
        for a in cand:
            S.slora_unload_adapter(dw.pool, a)
        return (t0.elapsed_time(td) if with_delta else None), t0.elapsed_time(tl), host_s

    for _ in range(2):
        fetch_round(False)
        fetch_round(True)
    alone = [fetch_round(False) for _ in range(steps)]
    both = [fetch_round(True) for _ in range(steps)]
    delta_ms = statistics.fmean(b[0] for b in both)
    load_ms = statistics.fmean(a[1] for a in alone)
    host_us = statistics.median(a[2] for a in alone) * 1e6
    load_ov_ms = statistics.fmean(b[1] for b in both)
    # the step alone, timed the same way (flush, then events on the launch stream)
    solo = []
    for _ in range(steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        flush()
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        solo.append(a.elapsed_time(b))
    solo_ms = statistics.fmean(solo)
    for a in cand:
        S.slora_load_adapter(dw.pool, a, int(w.ranks[a]), float(w.scales[a]))
    return {"adapters": len(cand), "bytes": nbytes,
            "ranks": np.bincount(w.ranks[cand]).nonzero()[0].tolist(),
            "host_enqueue_us": round(host_us, 1),
            "fetch_us_alone": round(load_ms * 1e3, 2),
            "h2d_GBps_alone": round(nbytes / (load_ms * 1e-3) / 1e9, 2),
            "fetch_us_with_step": round(load_ov_ms * 1e3, 2),
            "h2d_GBps_with_step": round(nbytes / (load_ov_ms * 1e-3) / 1e9, 2),
            "step_us_alone": round(solo_ms * 1e3, 2),
            "step_us_with_fetch": round(delta_ms * 1e3, 2),
            "step_slowdown": round(delta_ms / solo_ms - 1.0, 4),
            "timing": "HIP events: the step on the launch stream, the fetch on a second stream "
                      "that starts with the step; means over the timed steps, cache flushed "
                      "before each"}


def measure_forward(dw, w, steps, flush, stream):
    """The base product with the delta in the same tiles (slora_lora_forward:
    shrink, then one matrix-core kernel writing y = x W + s (x A) B) against
    the unfused alternative, the base product on hipBLASLt (torch.mm) followed
    by slora_lora_delta into its output; both with the workload's seeded dense
    base weight per projection, timed like the delta (flush before each step,
    HIP events on the launch stream), plus a dispatch-timed pass of the fused
    call (its kernels' own duration)."""
    import torch
    from rank_gemm_page_amd.hip_events import HipEvent
    spec = w.spec
    n_proj = spec.n_proj
    wts = [dw.base_weight(p) for p in range(n_proj)]
    w.drop_weight_cache()
    outs = [torch.empty(w.T, spec.h_out, dtype=dw.tdtype, device=dw.device) for _ in range(n_proj)]

    def fused():
        for p in range(n_proj):
            dw.forward(p, outs[p], stream=stream)

    def unfused():
        for p in range(n_proj):
            torch.mm(dw.x[spec.proj_x[p]], wts[p], out=outs[p])
            dw.delta(p, y=outs[p], stream=stream)

    def timed(run):
        for _ in range(3):
            flush()
            run()
        ts = []
        for _ in range(steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            flush()
            a.record(stream)
            run()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return statistics.fmean(ts)

    fused_ms = timed(fused)
    unfused_ms = timed(unfused)
    kev = [[(HipEvent(), HipEvent()) for _ in range(n_proj)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        flush()
        for p in range(n_proj):
            dw.forward_timed(p, outs[p], kev[k][p][0].handle, kev[k][p][1].handle, stream=stream)
    torch.cuda.synchronize()
    kern_ms = statistics.fmean(sum(kev[k][p][0].elapsed_ms(kev[k][p][1]) for p in range(n_proj))
                               for k in range(steps))
    sf, ef = dw.algorithmic_flops()
    base_flops = 2.0 * w.T * spec.h_in * spec.h_out
    flops = n_proj * (base_flops + sf + ef)
    e = 2 if spec.dtype == "f16" else 4
    tflops = flops / (kern_ms * 1e-3) / 1e12
    # algorithmic bytes of one call's base-plus-delta launches: x rows, W, the
    # batch's B pages, y written once
    fwd_bytes = e * (w.T * spec.h_in + spec.h_in * spec.h_out + int(dw.info["sum_rank"]) * spec.h_out
                     + w.T * spec.h_out)
    traffic, prof_us = load_traffic(spec.name, "forward_kernel", kind="forward")
    return {"roofline": {"bound": "mfma", "kernel": "shrink + forward_kernel", "achieved": round(tflops, 1),
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": traffic,
                         "algorithmic_bytes": fwd_bytes, "profiled_forward_kernels_us": prof_us},
            "ms_per_step": round(fused_ms, 5), "unfused_ms_per_step": round(unfused_ms, 5),
            "speedup_vs_unfused": round(unfused_ms / fused_ms, 3),
            "kernels_us_per_projection": round(kern_ms * 1e3 / n_proj, 3),
            "TFLOPs": round(flops / (kern_ms * 1e-3) / 1e12, 1),
            "mfma_frac_f16_peak": round(flops / (kern_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "flops_per_step": flops,
            "y_round_trip_saved_bytes": 2 * w.T * spec.h_out * n_proj * e,
            "method": "slora_lora_forward per projection vs torch.mm(x, W) + slora_lora_delta into "
                      "its output; seeded dense W; HIP events on the launch stream, cache flushed "
                      "before each step; kernels_us from dispatch-recorded events around the "
                      "shrink and the base-plus-delta kernel"}


def host_cpu_model():
    """The host CPU's model name (lscpu's "Model name", else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def measure_achievable(dw, w, launch_bytes, flush, stream, reps=5):
    """What the GPU delivers for one launch of the delta's size, cold, timed
    with dispatch-recorded events like the delta kernel: a contiguous streaming
    read of the launch's algorithmic bytes, and a gather (streaming hint) of as
    many whole page rows of the same pool as the launch reads adapter rows
    (random page ids of the same classes, so the same row sizes and the same
    scatter over the pool).  Each probe is the best of a few load depths."""
    import numpy as np
    import torch

    from rank_gemm_page_amd import slora as S
    from rank_gemm_page_amd.hip_events import HipEvent
    dev = dw.device
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    nbytes = (int(launch_bytes) + 15) // 16 * 16
    src = torch.ones(nbytes // 2, dtype=torch.int16, device=dev)

    def timed(launch):
        ms = []
        for _ in range(reps + 1):
            a, b = HipEvent(), HipEvent()
            flush()
            launch(a.handle, b.handle)
            b.synchronize()
            ms.append(a.elapsed_ms(b))
        return statistics.fmean(ms[1:])

    read = {}
    for items in (4, 8, 16):
        for nt in (False, True):
            read[(items, nt)] = timed(lambda a, b: S.slora_probe_read(src, nbytes, items, nt, sink, stream, a, b))
    (ri, rnt), rms = min(read.items(), key=lambda kv: kv[1])
    del src
    # the launch's adapter rows: sum_rank rows of A^T (class 0) and of B (the B class)
    r_u = int(dw.info["sum_rank"])
    rng = np.random.default_rng(1234)
    b_cls = 1 if w.spec.two_classes else 0
    e = 2 if w.spec.dtype == "f16" else 4
    arrays, gbytes, keep = [], 0, []
    for cls, n in ((0, r_u), (b_cls, r_u)):
        P = int(w.n_pages[cls])
        rows = torch.from_numpy(rng.choice(P, size=min(n, P), replace=False).astype(np.int32)).to(dev)
        keep.append(rows)
        rb = w.page_elems(cls) * e
        arrays.append((dw.pages[cls], rb, rb, rows, rows.numel()))
        gbytes += rows.numel() * rb
    gather = {}
    for items in (4, 8, 16):
        gather[items] = timed(lambda a, b: S.slora_probe_gather(arrays, items, sink, stream, a, b))
    gi, gms = min(gather.items(), key=lambda kv: kv[1])
    return {"stream_read_GBps": round(nbytes / (rms * 1e-3) / 1e9, 1), "stream_read_bytes": nbytes,
            "stream_read_us": round(rms * 1e3, 3), "stream_read_loads_in_flight": ri,
            "stream_read_nontemporal": rnt,
            "row_gather_GBps": round(gbytes / (gms * 1e-3) / 1e9, 1), "row_gather_bytes": gbytes,
            "row_gather_us": round(gms * 1e3, 3), "row_gather_loads_in_flight": gi,
            "method": "slora_probe_read / slora_probe_gather (one launch each, cache flushed "
                      "before each, dispatch-recorded HIP events, mean of "
                      f"{reps} after one untimed); best over 16-byte loads in flight per thread "
                      "{4, 8, 16} (and the streaming hint on or off for the read)"}


CONFIG_ORDER = ["decode7b", "tiny", "prefill7b", "mixed13b", "mlp70b"]


def measure_config(name, args, tuning, dev, headline):
    """One workload: the timed steps, the kernel's own duration, the roofline
    against 8 TB/s and against the achievable probes, and the CPU oracle."""
    import numpy as np
    import torch

    from rank_gemm_page_amd import slora as S
    from rank_gemm_page_amd.device_workload import DeviceWorkload
    from rank_gemm_page_amd.hip_events import HipEvent

    t_cfg = time.perf_counter()
    log(f"[bench] generating {name} seed={args.seed}")
    w = workload(name, args.seed, args.rank_pad)
    log(f"[bench] {name}: loading pool")
    dw = DeviceWorkload(w, dev, tuning=tuning)
    spec = w.spec
    n_proj = spec.n_proj
    info = dw.info
    log(f"[bench] {name}: T={w.T} segments={info['n_segments']} mfma_segments={info['n_mfma_segments']} "
        f"shrink_tiles={info['n_shrink_tiles']} expand_tiles={info['n_expand_tiles']} "
        f"(set up in {time.perf_counter() - t_cfg:.1f} s)")

    stream = torch.cuda.current_stream(dev)
    half = args.flush_mib * (1 << 20) // 2
    flush_src = torch.empty(max(half, 16), dtype=torch.uint8, device=dev)
    flush_dst = torch.empty_like(flush_src)
    flush_src.fill_(1)

    def flush():
        if args.flush_mib > 0:
            flush_dst.copy_(flush_src)

    # Several projections run as one launch (slora_lora_delta_multi) unless
    # --per-projection asks for one launch each.
    multi = n_proj > 1 and not args.staged and not args.per_projection

    def step(events=None, kev=None):
        if multi:
            if events is not None:
                events[0][0].record(stream)
            dw.delta_multi(stream=stream, events=None if kev is None else (kev[0][0].handle, kev[0][1].handle))
            if events is not None:
                events[0][2].record(stream)
            return
        for p in range(n_proj):
            if events is not None:
                events[p][0].record(stream)
            if args.staged:
                dw.shrink(p, stream=stream)
                if events is not None:
                    events[p][1].record(stream)
                dw.expand(p, stream=stream)
            elif kev is not None:
                # dispatch-recorded events: the kernel's own start and end
                dw.delta_timed(p, kev[p][0].handle, kev[p][1].handle, stream=stream)
            else:
                dw.delta(p, stream=stream)   # one fused launch per projection
            if events is not None:
                events[p][2].record(stream)

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_proj)]
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        flush()
        step(ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] {name}: {K} timed steps done in {wall * 1e3:.1f} ms wall (flushes included)")

    n_launch = 1 if multi else n_proj
    step_ms = [sum(ev[k][p][0].elapsed_time(ev[k][p][2]) for p in range(n_launch)) for k in range(K)]
    ms = statistics.fmean(step_ms)
    if args.staged:
        sh_ms = statistics.fmean(sum(ev[k][p][0].elapsed_time(ev[k][p][1]) for p in range(n_proj))
                                 for k in range(K))
        ex_ms = ms - sh_ms
        kern_ms = None
    else:
        # Second timed pass over the same steps: events recorded by the dispatch
        # itself give the fused kernel's own duration (what rocprofv3 reports);
        # recording them costs launch time, so this pass does not feed ms_per_step.
        kev = [[(HipEvent(), HipEvent()) for _ in range(n_proj)] for _ in range(K)]
        torch.cuda.synchronize()
        for k in range(K):
            flush()
            step(None, kev[k])
        torch.cuda.synchronize()
        for row in kev:
            row[-1][1].synchronize()
        kern_ms = [sum(kev[k][p][0].elapsed_ms(kev[k][p][1]) for p in range(n_launch))
                   for k in range(K)]
        log(f"[bench] {name}: {K} dispatch-timed steps done")
    assert S.slora_segments_read_error(dw.seg, stream) == 0, "a fused launch gave up waiting"

    # Host segment build and metadata upload, timed apart (PCIe-inclusive figures).
    builds = []
    for _ in range(20):
        t = time.perf_counter()
        seg = S.slora_build_segments(dw.pool, w.ids)
        builds.append(time.perf_counter() - t)
        S.slora_segments_destroy(seg)
    up_ms = []
    for _ in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dw.upload(stream)
        b.record(stream)
        b.synchronize()
        up_ms.append(a.elapsed_time(b))
    build_us = statistics.median(builds) * 1e6
    upload_us = statistics.median(up_ms) * 1e3

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            flush()
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    e = 2 if spec.dtype == "f16" else 4
    sb, eb = dw.algorithmic_bytes()
    sf, ef = dw.algorithmic_flops()
    launch_bytes = sb + eb        # one projection: its adapters' pages, x once, y read and written
    # One step's algorithmic bytes: every projection's pages and y, each distinct x once
    n_x = len(set(spec.proj_x))
    routed = int(info["n_routed"])
    step_bytes = n_proj * launch_bytes - (n_proj - n_x) * routed * spec.h_in * e
    flops = n_proj * (sf + ef)
    if args.staged:
        dominant = "shrink_kernel" if sh_ms >= ex_ms else "expand_kernel"
        dom_ms = max(sh_ms, ex_ms) / n_proj
        dom_bytes = sb if dominant == "shrink_kernel" else eb
        step_kern_ms = sh_ms + ex_ms
    elif multi:
        dominant = "fused_kernel"
        step_kern_ms = statistics.fmean(kern_ms)
        dom_ms = step_kern_ms            # one launch holds every projection
        dom_bytes = step_bytes
    else:
        dominant = "fused_kernel"
        step_kern_ms = statistics.fmean(kern_ms)
        dom_ms = step_kern_ms / n_proj
        dom_bytes = launch_bytes
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    traffic, profiled_us = load_traffic(name, dominant)
    value = routed / (ms * 1e-3)
    step_achieved = step_bytes / (step_kern_ms * 1e-3) / 1e9

    achievable = None
    if not args.no_probe and name != "tiny":
        log(f"[bench] {name}: achievable-bandwidth probes")
        achievable = measure_achievable(dw, w, launch_bytes, flush, stream)
    best = max(achievable["stream_read_GBps"], achievable["row_gather_GBps"]) if achievable else None

    out = {
        "ms_per_step": round(ms, 5),
        "value": round(value, 1),
        "unit": "tokens/s",
        "dtype": spec.dtype,
        "config": {"workload": name, "description": WORKLOAD_NOTES[name],
                   "tokens": routed, "h_in": spec.h_in, "h_out": spec.h_out,
                   "projections": n_proj, "distinct_x": n_x, "adapters": spec.n_adapters,
                   "segments": info["n_segments"], "mfma_segments": info["n_mfma_segments"],
                   "sum_rank": int(info["sum_rank"]), "seed": args.seed, "rank_pad": args.rank_pad,
                   "parallelism": "single GPU",
                   "tuning": {str(k): v for k, v in tuning.items()}},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": dom_bytes,
                     "avg_launch_us": round(dom_ms * 1e3, 3),
                     "profiled_avg_launch_us": round(profiled_us, 3) if profiled_us else None,
                     "achievable": achievable,
                     "frac_of_achievable": round(achieved / best, 4) if best else None},
        "step_roofline": {"algorithmic_bytes": step_bytes, "kernel_us": round(step_kern_ms * 1e3, 3),
                          "achieved": round(step_achieved, 1), "unit": "GB/s",
                          "frac": round(step_achieved / HBM_PEAK_GBPS, 4),
                          "frac_of_achievable": round(step_achieved / best, 4) if best else None,
                          "bytes": "per step: each projection's distinct adapter pages once, each "
                                   "distinct x once, every projection's y read and written"},
        "kernels": {**({"shrink_us": round(sh_ms * 1e3 / n_proj, 3),
                        "expand_us": round(ex_ms * 1e3 / n_proj, 3),
                        "shrink_GBps": round(sb / (sh_ms / n_proj * 1e-3) / 1e9, 1),
                        "expand_GBps": round(eb / (ex_ms / n_proj * 1e-3) / 1e9, 1)}
                       if args.staged else {"launch": ("fused, every projection in one launch "
                                                       "(slora_lora_delta_multi)") if multi
                                            else "fused (one kernel per projection)",
                                            "fused_kernel_us": round(dom_ms * 1e3, 3),
                                            "fused_step_us": round(ms * 1e3 / n_launch, 3)}),
                    "step_GBps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
                    "step_frac_hbm_peak": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "step_us_p10": round(float(np.percentile(step_ms, 10)) * 1e3, 3),
                    "step_us_p90": round(float(np.percentile(step_ms, 90)) * 1e3, 3),
                    "shrink_tiles": info["n_shrink_tiles"], "expand_tiles": info["n_expand_tiles"]},
        "host_build_us": round(build_us, 1),
        "metadata_upload_us": round(upload_us, 2),
        "metadata_bytes": int(info["meta_bytes"]),
        "wall_ms_per_step_incl_flush": round(wall * 1e3 / K, 4),
    }
    if kern_ms is not None:
        # the kernel's own duration per launch, spread over the timed steps
        per_launch = [k / (1 if multi else n_proj) * 1e3 for k in kern_ms]
        out["kernels"]["fused_kernel_us_median"] = round(statistics.median(per_launch), 3)
        out["kernels"]["fused_kernel_us_p10"] = round(float(np.percentile(per_launch, 10)), 3)
        out["kernels"]["fused_kernel_us_p90"] = round(float(np.percentile(per_launch, 90)), 3)
    # Matrix-core use: flops over the kernels' own time against the fp16 dense
    # peak, and against the attainable roofline min(peak, AI x 8 TB/s) at this
    # batch's arithmetic intensity.
    tflops = flops / (step_kern_ms * 1e-3) / 1e12
    ai = flops / step_bytes
    attainable = min(MFMA_F16_PEAK_TFLOPS, ai * HBM_PEAK_GBPS / 1e3)
    out["mfma"] = {"achieved_TFLOPs": round(tflops, 2), "peak_TFLOPs": MFMA_F16_PEAK_TFLOPS,
                   "frac_of_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 5),
                   "flops_per_step": flops, "arithmetic_intensity": round(ai, 3),
                   "attainable_TFLOPs": round(attainable, 2),
                   "frac_of_attainable": round(tflops / attainable, 4),
                   "note": "fp16 flops of the matrix-core and vector-ALU tiles together "
                           "(2 sum_t r_t (h_in + h_out) per projection)"}
    util = load_mfma_util(name)
    if util is not None:
        out["mfma"]["profiled"] = util
    if headline:
        if args.base_gemm:
            log("[bench] base x W products")
            out["base_gemm"] = measure_base_gemm(dw, w, K, flush, stream, ms)
        if args.forward:
            log("[bench] base product with the delta in the same tiles")
            out["forward"] = measure_forward(dw, w, K, flush, stream)
        if args.bmm_baseline:
            log("[bench] padded-BMM comparison path")
            out["bmm_path"] = measure_bmm_path(dw, w, K, flush, stream, ms)
        if args.prefetch > 0:
            log(f"[bench] adapter fetch: {args.prefetch} adapters per step")
            out["prefetch"] = measure_prefetch(dw, w, args.prefetch, K, flush, step, stream)
    dw.close()
    del dw, flush_src, flush_dst
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"[bench] {name}: timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, budget_s=10.0 if headline else 3.0, one_thread=headline)
        out["cpu_baseline"]["host_cpu_model"] = host_cpu_model()
    log(f"[bench] {name}: done in {time.perf_counter() - t_cfg:.1f} s")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all", choices=["all"] + CONFIG_ORDER,
                    help="all (default): decode7b as the headline, the other four under per_config")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="device copy between steps that evicts the last-level cache (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the achievable-bandwidth probes")
    ap.add_argument("--mfma-min-tokens", type=int, default=None)
    ap.add_argument("--gemv-expand-elems", type=int, default=None)
    ap.add_argument("--mfma-expand-cols", type=int, default=None)
    ap.add_argument("--mfma-shrink-splits", type=int, default=None)
    ap.add_argument("--xcds", type=int, default=None, help="XCD groups of the tile placement (1: none)")
    ap.add_argument("--tile-order", type=int, default=None,
                    help="0: tiles in adapter order, 1: clustered by rank, 2 (default): most bytes first")
    ap.add_argument("--fwd-group", type=int, default=None,
                    help="row blocks per group of the base-plus-delta tile order (0: automatic)")
    ap.add_argument("--fwd-tile", type=int, default=None, choices=[0, 32, 64, 128, 256],
                    help="base-plus-delta tile (0: automatic)")
    ap.add_argument("--shrink-rows", type=int, default=None,
                    help="rank rows per vector-ALU shrink tile (0: as many as fit)")
    ap.add_argument("--fwd-ksplit", type=int, default=None,
                    help="wave groups splitting a 32- or 64-row forward tile's steps (0: automatic)")
    ap.add_argument("--rank-pad", type=int, default=0,
                    help="round every adapter's rank up to a multiple of this (padded-rank comparison; 0: off)")
    ap.add_argument("--per-projection", action="store_true",
                    help="one fused launch per projection instead of one launch for all of them")
    ap.add_argument("--staged", action="store_true",
                    help="time the two stages as separate launches (slora_lora_shrink / _expand)")
    ap.add_argument("--prefetch", type=int, default=0, metavar="M",
                    help="also fetch M adapters the batch does not use from pinned host images "
                         "on a second stream, alone and while the step runs (slora_load_adapters_async)")
    ap.add_argument("--base-gemm", action="store_true",
                    help="also time the base products x W of the same step (torch.mm) for context")
    ap.add_argument("--forward", action="store_true",
                    help="also time the base product with the delta in the same tiles "
                         "(slora_lora_forward) against torch.mm + slora_lora_delta")
    ap.add_argument("--bmm-baseline", action="store_true",
                    help="also time the padded-BMM path (torch) on the same batch for comparison")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain copy of this size (PMC calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported; the delta shards by tokens or columns with no exchange, and "
              "bench.py measures one GPU's share.", file=sys.stderr, flush=True)
        sys.exit(3)

    import torch

    from rank_gemm_page_amd import slora as S

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tuning = {k: v for k, v in ((S.SLORA_TUNE_MFMA_MIN_TOKENS, args.mfma_min_tokens),
                                (S.SLORA_TUNE_GEMV_EXPAND_ELEMS, args.gemv_expand_elems),
                                (S.SLORA_TUNE_MFMA_EXPAND_COLS, args.mfma_expand_cols),
                                (S.SLORA_TUNE_MFMA_SHRINK_SPLITS, args.mfma_shrink_splits),
                                (S.SLORA_TUNE_XCDS, args.xcds),
                                (S.SLORA_TUNE_TILE_ORDER, args.tile_order),
                                (S.SLORA_TUNE_FWD_GROUP, args.fwd_group),
                                (S.SLORA_TUNE_FWD_TILE, args.fwd_tile),
                                (S.SLORA_TUNE_SHRINK_ROWS, args.shrink_rows),
                                (S.SLORA_TUNE_FWD_KSPLIT, args.fwd_ksplit))
              if v is not None}
    names = CONFIG_ORDER if args.config == "all" else [args.config]
    t_all = time.perf_counter()
    results = {n: measure_config(n, args, tuning, dev, headline=(i == 0)) for i, n in enumerate(names)}
    head = results[names[0]]
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        **{k: v for k, v in head.items() if k not in ("value", "unit", "ms_per_step", "dtype", "config",
                                                     "roofline")},
        "timing": "ms_per_step: HIP events recorded on the launch stream around each step's "
                  "delta launch(es); roofline.avg_launch_us: a second pass over as many steps "
                  "with HIP events recorded by the kernel dispatch itself "
                  "(slora_lora_delta_timed), the kernel's own duration as rocprofv3 reports "
                  "it; means over the timed steps; a "
                  f"{args.flush_mib} MiB device copy before every step evicts the 256 MB "
                  "last-level cache and is outside both",
    }
    if len(names) > 1:
        out["per_config"] = {n: results[n] for n in names[1:]}
    out["bench_wall_s"] = round(time.perf_counter() - t_all, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the cascade decode step on one MI355X.

Workload: shared prefix of 32768 tokens (one contiguous run of page-size-16 pages) plus 256
unique tokens per request in randomly permuted pages, batch 128, 32 heads x 128, fp16, q/k/v
~ N(0,1) * 0.5 -- the LLaMA2-7B-shaped setting of the "Cascade Inference" blog's evaluation.

One step = what a serving loop does per generated token for one layer: the CPU plan of the
step (load-balancing plan + level work lists, copied asynchronously to the device workspace)
and the cascade run (MFMA prefix kernel, suffix decode kernel, merge).  Inputs are resident in
HBM before the timed region.  Printed: one JSON line with the achieved algorithmic KV bytes/s
(prefix read once + every suffix), steps/s, the dominant kernel's roofline (HIP events around
each launch on the launch stream), HBM traffic from rocprofv3 counters when profiles/ holds
them for the current kernel sources, and the fp64 CPU oracle timed on a bounded sample.

Also reported, outside the timed steps: the distribution of single-run device times (back to
back, and with the last-level cache evicted before each run); the same step without the
cascade (every request reads the shared prefix through its own full page list) with the
largest output difference between the two; the in-place append of one token per request; and
the LLaMA2-7B decode shape (64 x 4096 tokens) over fp16 pools and over FP8 E4M3 pools; and
the same cascade step over FP8 E4M3 pools; a causal prefill of ragged multi-token queries
(matrix-core TFLOP/s); and the load-balanced split-KV decode with grouped heads (256 requests,
32 / 8 heads, bf16, log-uniform lengths 128..32768).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV bytes/s from HBM (% of peak) + decode steps/s, cascade 32K prefix, batch 128"
PEAK_HBM_GBPS = 8000.0
PEAK_FP16_MFMA_TFLOPS = 2500.0   # dense fp16 matrix-core peak of the MI355X
KERNEL_SOURCES = ["paged_kv_cascade_amd/csrc/prefix_kernel.h", "paged_kv_cascade_amd/csrc/decode.hip",
                  "paged_kv_cascade_amd/csrc/decode_kernel.h", "paged_kv_cascade_amd/csrc/merge.hip",
                  "paged_kv_cascade_amd/csrc/merge_ops.h", "paged_kv_cascade_amd/csrc/device_common.h",
                  "paged_kv_cascade_amd/csrc/kernels.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cascade32k_b128_hbm_traffic.json")
# FETCH_SIZE of one non-cascade step over the same data (rocprofv3, scaled by the copy
# calibration), from the committed counter summary of that kernel.
NONCASCADE_FETCH_BYTES = None


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=0,
                    help="requests of the CPU oracle sample (all 32 heads each); 0: the whole step")
    ap.add_argument("--cpu-baseline-only", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--copy-calib", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration under rocprofv3)")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


class Step:
    """Buffers and per-step calls of the serving loop: the CPU plan of the step into one of
    two pinned host buffers, then the cascade run launched on the stream (`__call__`; the plan
    is built with defer_upload, so the run's level kernel reads its items from the host buffer
    and copies the plan into the one device workspace, with no separate upload launch), or the
    upload of the plan on the stream and the replay of the run captured once in a HIP graph
    (`step_graph`; FlashInfer paper summary, section A3: plan on the CPU outside the graph,
    run captured; appendix D: fixed pointers).  Both compute the same bits (checked in main).
    On this stack a graph replay costs the GPU about 6-7 us per step more than the direct
    launches, so the timed loop launches directly."""

    def __init__(self, api, w, capture=True):
        import torch
        self.api, self.w = api, w
        self.levels = api.HostLevels([{"qo_indptr": lv["qo_indptr"], "kv_lens": lv["kv_lens"]} for lv in w.levels])
        shape = (w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
        self.params = api.make_params(*shape)
        self.params_deferred = api.make_params(*shape, defer_upload=True)   # same layout
        # Two pinned host buffers used alternately: the CPU may write step i+1's plan while
        # step i still reads (or copies) its own.  One device workspace (fixed pointers).
        self.ws = [api.Workspace(self.params, self.levels) for _ in range(2)]
        for k in (1,):
            self.ws[k].device = self.ws[0].device
        self.copy_done = [None, None]
        self.kv_lens = w.cache_seqlens.cpu().to(torch.int32).contiguous()
        self.devs, self.keep = [], []
        for lv in w.levels:
            d, k = api.level_dev(lv)
            self.devs.append(d)
            self.keep.append(k)
        self.out = torch.empty_like(w.q)
        self.lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")
        self.i = 0
        self.info = self.plan()
        self.mark()
        self.graph = None
        if capture:
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    self.run(self.info)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            self.graph = g

    def plan(self, deferred=False):
        """The step's plan into the next host buffer, once the work that read it two steps ago
        has completed (a deferred plan is read by the run, so mark() follows the run)."""
        k = self.i % 2
        if self.copy_done[k] is not None:
            self.copy_done[k].synchronize()
        info = self.api.plan(self.params_deferred if deferred else self.params, self.kv_lens, self.levels,
                             workspace=self.ws[k])
        self.i += 1
        self.k = k
        return info

    def mark(self):
        """The host buffer of the latest plan may be rewritten once the work enqueued so far is done."""
        import torch
        ev = torch.cuda.Event()
        ev.record()
        self.copy_done[self.k] = ev

    def run(self, info):
        """The cascade run itself, launched eagerly (per-kernel timing needs eager launches)."""
        w = self.w
        self.api.cascade_decode(info, w.q, w.k_pool, w.v_pool, self.devs, w.block_table, w.cache_seqlens,
                                sm_scale=w.sm_scale, out=self.out, lse=self.lse)

    def replay(self):
        """The captured run (the workspace holds the latest plan)."""
        self.graph.replay()

    def __call__(self):
        """One serving-loop step: the plan, then the cascade run that brings it over (direct
        launches)."""
        self.run(self.plan(deferred=True))
        self.mark()

    def step_graph(self):
        """The same step with the plan uploaded on the stream and the run replayed from the
        captured graph."""
        self.plan()
        self.replay()
        self.mark()


def cpu_oracle_baseline(n_req):
    """The fp64 oracle (one softmax over each request's 33,024 gathered tokens, every head) on
    requests of the same workload generated on the host, one worker process per core this
    process may run on, at most 16 (a one-GPU machine's CPU share; BLAS pinned to one thread per
    worker); n_req = 0: all 128 requests of the step (about 10 s on 16 cores), else a sample
    scaled to the step.  Runs in a process that never touches the GPU."""
    import multiprocessing as mp

    import numpy as np

    from paged_kv_cascade_amd import workloads

    w = workloads.cascade_two_level(device="cpu")
    alg_bytes = w.algorithmic_kv_bytes()
    global _CPU_CTX
    _CPU_CTX = (w.q.float().double().numpy(), w.k_pool.numpy(), w.v_pool.numpy(), w.page_size,
                w.sm_scale, w.levels, w.block_table.numpy(), w.cache_seqlens.numpy())
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cores = max(1, min(16, avail))
    if n_req <= 0:
        n_req = w.batch
    reqs = list(range(0, w.batch, max(1, w.batch // n_req)))[:n_req]
    cores = min(cores, len(reqs))
    walls = []
    with mp.get_context("fork").Pool(cores, initializer=_cpu_worker_init) as pool:
        for _ in range(3):
            t0 = time.perf_counter()
            outs = pool.map(_cpu_one_request, reqs)
            walls.append(time.perf_counter() - t0)
            assert all(np.all(np.isfinite(o)) for o in outs)
    dt = sorted(walls)[1]   # median of three passes
    step_s = dt * w.batch / len(reqs)
    return {"value": round(alg_bytes / step_s / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "steps_per_s": round(1.0 / step_s, 5), "seconds_per_step": round(step_s, 3),
            "host_cores": os.cpu_count(), "cores_available": avail,
            "pass_seconds": [round(x, 3) for x in walls],
            "sample": f"{len(reqs)} of {w.batch} requests x all {w.num_qo_heads} heads "
                      f"(33,024 tokens each) in {dt:.1f} s wall (median of 3 passes) on {cores} worker processes "
                      f"({avail} cores available to the process, at most 16 used)"
                      + ("" if len(reqs) == w.batch else f", scaled to one {w.batch}-request step")}


_CPU_CTX = None


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_one_request(b):
    from oracle import attention as oatt
    q, k, v, P, scale, levels, bt, sl = _CPU_CTX
    O, L = oatt.cascade_decode(q, k, v, P, scale, levels, bt, sl, requests=[b])
    return O[b]


def device_record(api):
    """The device the run used: name, architecture, compute units, HIP version, and its GFX and
    memory clocks read (read-only) through amdsmi, matched to this device by PCI bus; the clocks
    are null when amdsmi is missing or the device cannot be matched."""
    import torch
    props = torch.cuda.get_device_properties(0)
    rec = {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
           "compute_units": api.device_info(0)["num_cus"], "hip_version": torch.version.hip,
           "clocks_mhz": None}
    bus = getattr(props, "pci_bus_id", None)
    if bus is None:
        return rec
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        try:
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if int(bdf.split(":")[1], 16) != int(bus):
                    continue
                g = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                m = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)
                rec["clocks_mhz"] = {"gfx_now": g.get("clk"), "gfx_max": g.get("max_clk"),
                                     "mem_now": m.get("clk"), "mem_max": m.get("max_clk"), "bdf": bdf}
                break
        finally:
            amdsmi.amdsmi_shut_down()
    except Exception:
        rec["clocks_mhz"] = None
    return rec


def run_cpu_baseline_child(n_req):
    """Starts the CPU-oracle leg as a child process (before this process uses the GPU)."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
                        "--cpu-requests", str(n_req)], capture_output=True, text=True, timeout=900)
    if r.returncode != 0:
        print(r.stderr[-2000:], file=sys.stderr, flush=True)
        return None
    return json.loads(r.stdout.strip().splitlines()[-1])


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 2), "p50": round(float(np.percentile(a, 50)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def step_time_distribution(step, n, evict=None):
    """Device time of n single cascade runs (direct launches of the latest plan), each between
    its own pair of events on the launch stream; with `evict`, a 512 MiB buffer is rewritten
    before each run, outside the pair, so the run starts with none of its KV in the
    last-level cache."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        if evict is not None:
            evict.add_(1)
        a.record()
        step.run(step.info)
        b.record()
    torch.cuda.synchronize()
    return percentiles([1e3 * a.elapsed_time(b) for a, b in evs])


def noncascade_comparison(api, w, step, info, runs=5):
    """The same step without the cascade: every request attends over its own full page list
    (the 2048 prefix pages then its 16 suffix pages, 33,024 tokens) through the batch decode
    kernel, so each request reads the shared prefix itself.  Returns its time, its algorithmic
    KV bytes, the cascade's speedup over it and the largest output difference between the two."""
    import torch
    pre = torch.tensor(w.levels[0]["kv_page_indices"], dtype=torch.int32, device="cuda")
    bt = torch.cat([pre.unsqueeze(0).expand(w.batch, -1), w.block_table], dim=1).contiguous()
    lens = (w.cache_seqlens + w.levels[0]["kv_lens"][0]).to(torch.int32)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")
    api.batch_decode_paged(w.q, w.k_pool, w.v_pool, bt, lens, sm_scale=w.sm_scale, out=out, lse=lse)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(runs):
        api.batch_decode_paged(w.q, w.k_pool, w.v_pool, bt, lens, sm_scale=w.sm_scale, out=out, lse=lse)
    b.record()
    step.run(info)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / runs
    nbytes = int(lens.sum()) * w.num_kv_heads * w.head_dim * 2 * w.esize
    d_o = float((out.float() - step.out.float()).abs().max())
    d_l = float((lse - step.lse).abs().max())
    # Its requests re-read one prefix, so part of the algorithmic bytes come from the caches
    # (the counters fetch less than the algorithmic total from HBM): the rate below is
    # algorithmic bytes over time, cache-assisted, not an HBM rate.
    return {"ms_per_step": round(ms, 4), "alg_kv_bytes_per_step": nbytes,
            "alg_bytes_per_s_GB_cache_assisted": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_fetch_bytes_per_step_counters": NONCASCADE_FETCH_BYTES, "runs": runs,
            "max_abs_diff_vs_cascade": {"o": d_o, "lse": d_l}}


def gqa_decode_timing(api, workloads, runs=20):
    """Load-balanced split-KV decode with grouped heads: 256 requests, 32 query / 8 KV heads,
    bf16, lengths log-uniform in [128, 32768], through the plan over #CTA = 2 x compute units
    (alpha = beta = 1) and over the library's default #CTA; algorithmic bytes = every request's
    K and V once."""
    import torch
    w = workloads.gqa_split(device="cuda")
    lens = w.cache_seqlens.cpu().tolist()
    alg = sum(lens) * w.num_kv_heads * w.head_dim * 2 * w.esize
    cus = api.device_info(0)["num_cus"]
    o = torch.empty_like(w.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")
    out = {"workload": w.name, "alg_bytes": alg}
    for name, nc in (("plan_2x_cus", 2 * cus), ("plan_default", 0)):
        params = api.make_params(w.batch, w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                 num_ctas=nc, alpha=1, beta=1)
        ws = api.Workspace(params)
        info = api.plan(params, lens, workspace=ws)

        def run():
            api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                   sm_scale=w.sm_scale, plan_info=info, out=o, lse=lse)

        for _ in range(5):
            run()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(runs):
            run()
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / runs
        out[name] = {"num_ctas": info.num_ctas, "items": info.dec_items, "merged_requests": info.num_merge,
                     "us_per_run": round(us, 1), "alg_GBps": round(alg / us / 1e3, 1),
                     "frac_of_peak": round(alg / us / 1e3 / PEAK_HBM_GBPS, 4)}
    del w
    torch.cuda.empty_cache()
    return out


def fp8_decode_comparison(api, workloads, runs=10):
    """Batch decode of the LLaMA2-7B decode shape (64 requests x 4096 tokens, 32 heads x 128,
    page 16, fp16 queries) over fp16 pools and over the same pools quantised to FP8 E4M3:
    KV kernel time and algorithmic KV bytes/s of each (HIP events around each launch)."""
    import torch
    w = workloads.paged_decode(batch=64, kv_len=4096, page_size=16, dtype=torch.float16, device="cuda")
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.25)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.25)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")
    tokens = int(w.cache_seqlens.sum())
    res = {"workload": w.name}
    for name, fn, es in (
            ("fp16", lambda: api.batch_decode_paged(w.q, w.k_pool, w.v_pool, w.block_table, w.cache_seqlens,
                                                    sm_scale=w.sm_scale, out=out, lse=lse), 2),
            ("fp8_e4m3", lambda: api.batch_decode_paged_fp8(w.q, k8, v8, w.block_table, w.cache_seqlens,
                                                            k_scale=0.25, v_scale=0.25, sm_scale=w.sm_scale,
                                                            out=out, lse=lse), 1)):
        fn()
        torch.cuda.synchronize()
        api.timing_reset()
        api.timing_enable(True)
        for _ in range(runs):
            fn()
        torch.cuda.synchronize()
        n, ms = api.timing_read(api.KIND_DECODE)
        api.timing_enable(False)
        us = 1e3 * ms / max(1, n)
        nbytes = tokens * w.num_kv_heads * w.head_dim * 2 * es
        res[name] = {"avg_us": round(us, 1), "alg_bytes": nbytes, "achieved_GBps": round(nbytes / us / 1e3, 1),
                     "frac_of_peak": round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4)}
    res["speedup_fp8_over_fp16"] = round(res["fp16"]["avg_us"] / res["fp8_e4m3"]["avg_us"], 3)
    del w, k8, v8
    torch.cuda.empty_cache()
    return res


def fp8_cascade_timing(api, workloads, w, step, info, runs=50):
    """The same cascade step over the workload's pools quantised to FP8 E4M3 (k_scale = v_scale =
    0.25, fp16 queries): device time per run with the step's plan, per-kernel times, and its
    algorithmic KV bytes/s (one byte per element) -- against the fp16 run of the same plan."""
    import torch
    k8 = workloads.fp8_e4m3_pool(w.k_pool, 0.25)
    v8 = workloads.fp8_e4m3_pool(w.v_pool, 0.25)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.batch, w.num_qo_heads, dtype=torch.float32, device="cuda")

    def run():
        api.cascade_decode_fp8(info, w.q, k8, v8, step.devs, w.block_table, w.cache_seqlens, k_scale=0.25,
                               v_scale=0.25, sm_scale=w.sm_scale, out=out, lse=lse)

    for _ in range(10):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(runs):
        run()
    b.record()
    torch.cuda.synchronize()
    us = 1e3 * a.elapsed_time(b) / runs
    api.timing_reset()
    api.timing_enable(True)
    for _ in range(runs):
        run()
    torch.cuda.synchronize()
    kern = {}
    for kind, name in ((api.KIND_PREFIX, "prefix_mfma"), (api.KIND_DECODE, "suffix_decode")):
        n, ms = api.timing_read(kind)
        kern[name] = round(1e3 * ms / max(1, n), 2)
    api.timing_enable(False)
    nbytes = w.algorithmic_kv_bytes() // w.esize
    del k8, v8
    torch.cuda.empty_cache()
    return {"us_per_run": round(us, 1), "alg_kv_bytes_per_step": nbytes,
            "alg_GBps": round(nbytes / us / 1e3, 1), "kernel_avg_us": kern, "runs": runs}


def prefill_timing(api, runs=10):
    """Ragged multi-token queries at LLaMA2-7B head shape: 8 requests of 2048 new tokens over
    2048-token sequences (self-attention prefill), causal, fp16, page 16, level #CTA 64.  The
    level kernel is matrix-core work: reported in TFLOP/s of the visible (query, key) pairs,
    4 * D * Hq flops each, against the dense fp16 peak."""
    import torch
    B, lq, lkv, H, D, P = 8, 2048, 2048, 32, 128, 16
    npg = lkv // P
    g = torch.Generator().manual_seed(1006)
    bt = torch.randperm(B * npg, generator=g).to(torch.int32).view(B, npg).contiguous().cuda()
    dg = torch.Generator(device="cuda").manual_seed(1007)
    q = (torch.randn(B * lq, H, D, generator=dg, device="cuda") * 0.5).half()
    k = (torch.randn(B * npg, P, H, D, generator=dg, device="cuda") * 0.5).half()
    v = (torch.randn(B * npg, P, H, D, generator=dg, device="cuda") * 0.5).half()
    qi = torch.arange(0, (B + 1) * lq, lq, dtype=torch.int32, device="cuda")
    kvl = torch.full((B,), lkv, dtype=torch.int32, device="cuda")
    info, ws, _ = api.prefill_plan([lq] * B, [lkv] * B, H, H, D, P, level_ctas=64, causal=True)
    out = torch.empty_like(q)
    lse = torch.empty(B * lq, H, dtype=torch.float32, device="cuda")

    def run():
        api.batch_prefill_paged(info, q, k, v, bt, qi, kvl, causal=True, out=out, lse=lse)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    api.timing_reset()
    api.timing_enable(True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(runs):
        run()
    b.record()
    torch.cuda.synchronize()
    n, ms = api.timing_read(api.KIND_PREFIX)
    nm, msm = api.timing_read(api.KIND_MERGE_PLAN)
    api.timing_enable(False)
    pairs = B * lq * (lq + 1) // 2          # visible (query, key) pairs, causal
    flops = 4.0 * D * H * pairs
    kus = 1e3 * ms / max(1, n)
    res = {"workload": f"prefill_causal_b{B}_q{lq}_kv{lkv}_h{H}_d{D}_p{P}_f16", "us_per_run": round(1e3 * a.elapsed_time(b) / runs, 1),
           "level_kernel_us": round(kus, 1), "merge_us": round(1e3 * msm / max(1, nm), 1),
           "flops": flops, "level_kernel_TFLOPs": round(flops / kus / 1e6, 1),
           "frac_of_fp16_mfma_peak": round(flops / kus / 1e6 / 2500.0, 4)}
    del q, k, v, out
    torch.cuda.empty_cache()
    return res


def append_timing(api, w, runs=50):
    """Appending one new K/V token per request (the step before decode) for the cascade
    workload's batch and head shape: 128 requests with 256 cached suffix tokens each and a
    17th page already allocated, in pools of their own.  Device time per call."""
    import torch
    P, B = w.page_size, w.batch
    npg = w.block_table.shape[1] + 1
    shape = (B * npg, P, w.num_kv_heads, w.head_dim)
    kp = torch.zeros(shape, dtype=w.dtype, device="cuda")
    vp = torch.zeros_like(kp)
    bt = torch.arange(B * npg, dtype=torch.int32, device="cuda").view(B, npg)
    lens = w.cache_seqlens.clone()
    new_lens = torch.empty_like(lens)
    k_new = torch.ones(B, w.num_kv_heads, w.head_dim, dtype=w.dtype, device="cuda")
    v_new = torch.ones_like(k_new)
    api.append_kv(k_new, v_new, kp, vp, bt, lens, new_seqlens=new_lens)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(runs):
        api.append_kv(k_new, v_new, kp, vp, bt, lens, new_seqlens=new_lens)
    b.record()
    torch.cuda.synchronize()
    written = int((kp[:, 0] != 0).any(dim=-1).any(dim=-1).sum())
    res = {"avg_us": round(1e3 * a.elapsed_time(b) / runs, 2), "tokens_per_call": B,
           "bytes_written_per_call": 2 * B * w.num_kv_heads * w.head_dim * w.esize,
           "pages_written": written}
    del kp, vp
    torch.cuda.empty_cache()
    return res


def three_level_timing(api, workloads, runs=50):
    """The multi-level cascade: a 16384-token global prefix, 4 groups of 32 requests with a
    4096-token group prefix each, 512 unique tokens per request (batch 128, 32 heads x 128,
    fp16, page 16, every page placed by a seeded permutation).  Device time per run (back to
    back, and with the last-level cache evicted first), per-kernel averages from HIP events
    around each launch, and each kernel's algorithmic KV bytes per launch: 268,435,456 for
    each level (16384 tokens of the global prefix; 4 x 4096 tokens of group prefixes) and
    1,073,741,824 for the suffix decode (128 x 512 tokens); 1,610,612,736 per run."""
    import torch
    w = workloads.cascade_multi_level(device="cuda")
    st = Step(api, w)
    alg = w.algorithmic_kv_bytes()
    per_tok = w.num_kv_heads * w.head_dim * 2 * w.esize
    lvl_bytes = [sum(lv["kv_lens"]) * per_tok for lv in w.levels]
    suf_bytes = alg - sum(lvl_bytes)
    for _ in range(10):
        st()
    torch.cuda.synchronize()
    api.timing_reset()
    api.timing_enable(True)
    for _ in range(runs):
        st.run(st.info)
    torch.cuda.synchronize()
    kern = {}
    n, ms = api.timing_read(api.KIND_PREFIX)
    kern["level_mfma"] = {"launches": n, "avg_us": round(1e3 * ms / max(1, n), 2),
                          "alg_bytes_per_launch": lvl_bytes[0]}
    n, ms = api.timing_read(api.KIND_DECODE)
    kern["suffix_decode"] = {"launches": n, "avg_us": round(1e3 * ms / max(1, n), 2), "alg_bytes_per_launch": suf_bytes}
    n, ms = api.timing_read(api.KIND_MERGE_PLAN)
    kern["merge"] = {"launches": n, "avg_us": round(1e3 * ms / max(1, n), 2)}
    api.timing_enable(False)
    for name in ("level_mfma", "suffix_decode"):
        k = kern[name]
        k["achieved_GBps"] = round(k["alg_bytes_per_launch"] / (k["avg_us"] * 1e-6) / 1e9, 1)
        k["frac_of_peak"] = round(k["achieved_GBps"] / PEAK_HBM_GBPS, 4)
    warm = step_time_distribution(st, runs)
    evict = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    cold = step_time_distribution(st, min(runs, 30), evict)
    del evict
    t0 = time.perf_counter()
    for _ in range(runs):
        st()
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / runs
    res = {"workload": w.name, "alg_kv_bytes_per_step": alg, "floor_us_at_peak": round(alg / PEAK_HBM_GBPS / 1e3, 1),
           "ms_per_step": round(ms_step, 4), "alg_GBps": round(alg / (ms_step * 1e-3) / 1e9, 1),
           "frac_of_peak": round(alg / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
           "device_us_per_run": {"back_to_back": warm, "llc_evicted": cold}, "kernels": kern, "runs": runs}
    del st, w
    torch.cuda.empty_cache()
    return res


def load_traffic(src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when it is
    missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t


def read_stream_peak(api):
    """The device's achievable read rate: one nontemporal 16-byte-load stream over 2 GiB."""
    import torch
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = api.read_stream_probe(buf)
    for _ in range(2):
        api.read_stream_probe(buf, sink)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(10):
        api.read_stream_probe(buf, sink)
    ev1.record()
    torch.cuda.synchronize()
    gbps = buf.numel() / (ev0.elapsed_time(ev1) / 10 * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    return gbps


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}), flush=True)
        sys.exit(2)
    if args.cpu_baseline_only:
        print(json.dumps(cpu_oracle_baseline(args.cpu_requests)), flush=True)
        return
    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu oracle baseline (child process, host only) ...", file=sys.stderr, flush=True)
        cpu = run_cpu_baseline_child(args.cpu_requests)
    import torch

    if args.copy_calib:
        copy_calibration()
        return
    from paged_kv_cascade_amd import api, workloads

    t_setup = time.perf_counter()
    w = workloads.cascade_two_level(device="cuda")
    alg_bytes = w.algorithmic_kv_bytes()                  # 1,073,741,824
    prefix_bytes = sum(w.levels[0]["kv_lens"]) * w.num_kv_heads * w.head_dim * 2 * w.esize
    suffix_bytes = alg_bytes - prefix_bytes
    step = Step(api, w)
    torch.cuda.synchronize()
    print(f"# setup {time.perf_counter() - t_setup:.1f}s; workload {w.name}; "
          f"{alg_bytes} algorithmic KV bytes per step", file=sys.stderr, flush=True)

    # As a serving process does once it is set up: move the objects that live for the whole
    # run out of the collector's reach, so that a full collection (tens of ms with torch
    # loaded) cannot land inside the loop, and keep the collector off while steps are timed.
    gc.collect()
    gc.freeze()

    # The replayed graph computes what the eager run computes (same kernels, same plan).
    step.step_graph()
    torch.cuda.synchronize()
    ref_o, ref_l = step.out.clone(), step.lse.clone()
    step.run(step.info)
    torch.cuda.synchronize()
    graph_equal = bool(torch.equal(ref_o, step.out) and torch.equal(ref_l, step.lse))

    # An idle GPU comes back at lower clocks and takes tens of milliseconds of steady work to
    # reach the serving loop's again (in a kernel trace the first ~80 level-kernel launches
    # after start-up average 115-127 us, later ones 100 us): replays first, untimed.
    for _ in range(200):
        step.run(step.info)
    torch.cuda.synchronize()
    evict = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    dist_cold = step_time_distribution(step, 50, evict)
    del evict
    dist_warm = step_time_distribution(step, max(100, args.steps))

    # W warm-up steps, right after the GPU work above (no idle gap before the timed steps).
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly K serving-loop steps (plan on the CPU and its upload, then the run).
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    ms_step = 1e3 * elapsed / args.steps

    # The same K steps with the run replayed from the captured graph.
    for _ in range(20):
        step.step_graph()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.step_graph()
    torch.cuda.synchronize()
    ms_step_graph = 1e3 * (time.perf_counter() - t0) / args.steps

    # Device-only steps (one plan, K runs; then K graph replays) -- the kernels alone.
    step.plan()
    step.mark()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run(step.info)
    torch.cuda.synchronize()
    ms_dev = 1e3 * (time.perf_counter() - t0) / args.steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.replay()
    torch.cuda.synchronize()
    ms_dev_graph = 1e3 * (time.perf_counter() - t0) / args.steps

    # Per-kernel durations: HIP events the library records around each launch on its stream
    # (eager launches), taken right after the timed and device-only steps, at the clocks the
    # serving loop runs at.
    api.timing_reset()
    api.timing_enable(True)
    n_kern = max(100, args.steps)
    for _ in range(n_kern):
        step.run(step.info)
    torch.cuda.synchronize()
    kern = {}
    for kind, name in ((api.KIND_PREFIX, "prefix_mfma"), (api.KIND_DECODE, "suffix_decode"),
                       (api.KIND_MERGE_PLAN, "merge")):
        n, ms = api.timing_read(kind)
        kern[name] = {"launches": n, "avg_us": round(1e3 * ms / max(1, n), 2)}
    api.timing_enable(False)
    kern["prefix_mfma"]["alg_bytes"] = prefix_bytes
    kern["suffix_decode"]["alg_bytes"] = suffix_bytes
    for name in ("prefix_mfma", "suffix_decode"):
        k = kern[name]
        k["achieved_GBps"] = round(k["alg_bytes"] / (k["avg_us"] * 1e-6) / 1e9, 1)
        k["frac_of_peak"] = round(k["achieved_GBps"] / PEAK_HBM_GBPS, 4)

    # The device, with its clocks right after the steady-state kernel timing.
    device = device_record(api)

    # The plan's CPU time alone, as the timed steps build it (deferred: no GPU work; the GPU
    # idles meanwhile, so it comes after the GPU timings).
    t0 = time.perf_counter()
    for _ in range(200):
        step.plan(deferred=True)
    ms_plan = 1e3 * (time.perf_counter() - t0) / 200
    torch.cuda.synchronize()

    dom = max(("prefix_mfma", "suffix_decode"), key=lambda n: kern[n]["avg_us"])
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash)
    roof = {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["achieved_GBps"], "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": kern[dom]["frac_of_peak"],
            "traffic": (traffic or {}).get(dom, {}).get("hbm_bytes_per_launch") if traffic else None,
            "alg_bytes_per_launch": kern[dom]["alg_bytes"], "avg_launch_us": kern[dom]["avg_us"]}

    # The level kernel's matrix-core work: S^T = K Q^T and O^T += V^T P^T, 2 * head_dim flops
    # each per (query, prefix token, head): 4 * 128 * 32768 * 32 * 128 = 68,719,476,736 per launch.
    prefix_flops = 4 * w.head_dim * sum(w.levels[0]["kv_lens"]) * w.num_qo_heads * w.batch
    pk = kern["prefix_mfma"]
    mfma = {"kernel": "prefix_mfma", "flops_per_launch": prefix_flops,
            "achieved_TFLOPs": round(prefix_flops / (pk["avg_us"] * 1e-6) / 1e12, 1),
            "peak_TFLOPs": PEAK_FP16_MFMA_TFLOPS,
            "frac": round(prefix_flops / (pk["avg_us"] * 1e-6) / 1e12 / PEAK_FP16_MFMA_TFLOPS, 4),
            "busy_frac_counters": (traffic or {}).get("prefix_mfma", {}).get("mfma_busy_frac") if traffic else None}
    if mfma["busy_frac_counters"] is not None:
        mfma["busy_frac_counters"] = round(mfma["busy_frac_counters"], 4)

    info = step.info
    nonc = noncascade_comparison(api, w, step, info)
    if traffic and "noncascade_decode_full_tables" in traffic:
        nonc["hbm_fetch_bytes_per_step_counters"] = traffic["noncascade_decode_full_tables"]["hbm_read_bytes"]
    nonc["cascade_speedup"] = round(nonc["ms_per_step"] / (dist_warm["p50"] * 1e-3), 2)
    app = append_timing(api, w)
    fp8c = fp8_cascade_timing(api, workloads, w, step, info)
    del step, w
    torch.cuda.empty_cache()
    three = three_level_timing(api, workloads)
    pre = prefill_timing(api)
    fp8 = fp8_decode_comparison(api, workloads)
    gqa = gqa_decode_timing(api, workloads)
    stream_gbps = read_stream_peak(api)
    for name in ("prefix_mfma", "suffix_decode"):
        kern[name]["frac_of_read_stream_peak"] = round(kern[name]["achieved_GBps"] / stream_gbps, 4)

    value = alg_bytes / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "cascade_prefix32768_suffix256_b128_h32_d128_p16", "batch": 128,
                   "prefix_len": 32768, "suffix_len": 256, "heads": 32, "head_dim": 128,
                   "page_size": 16, "alg_kv_bytes_per_step": alg_bytes},
        "steps_per_s": round(1e3 / ms_step, 1),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBPS, 2),
        "step": "CPU plan into a pinned buffer + its upload, then the cascade run (level kernel, "
                "suffix kernel with the merge in the same launch) launched on the stream",
        "graph_replay_equals_eager_run": graph_equal,
        "graph_replay_loop": {"ms_per_step": round(ms_step_graph, 4),
                              "steps_per_s": round(1e3 / ms_step_graph, 1),
                              "ms_per_step_device_only": round(ms_dev_graph, 4)},
        "read_stream_peak_GBps": round(stream_gbps, 1),
        "pct_of_read_stream_peak": round(100 * value / stream_gbps, 2),
        "ms_per_step_device_only": round(ms_dev, 4),
        "ms_plan_cpu": round(ms_plan, 4),
        "device_us_per_run": {"back_to_back": dist_warm, "llc_evicted": dist_cold},
        # The same algorithmic bytes over the median run with the last-level cache evicted first
        # (no reuse of the previous step's reads): the cold-cache rate of the cascade run.
        "llc_evicted_alg_GBps": round(alg_bytes / (dist_cold["p50"] * 1e-6) / 1e9, 1),
        "kernels": kern,
        "roofline": roof,
        "prefix_mfma_utilisation": mfma,
        "device": device,
        "three_level_cascade": three,
        "noncascade_same_step": nonc,
        "append_kv": app,
        "fp8_kv_decode": fp8,
        "gqa_split_decode": gqa,
        "fp8_kv_cascade": fp8c,
        "prefill": pre,
        "kernel_source_hash": src_hash,
    }
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the RESOLVE hot path on one MI355X.

A step is one decode step through every layer of the workload: for each
layer, one hisparse_resolve over all requests (hash build, cache probe,
victim choice, metadata update, host fetch of the misses, publication).
Inputs (the whole selection trace and the pinned host pool) are resident
before the timed region starts.  The default workload is the largest
single-GPU configuration, gqa_record (64 requests x 16 layers, 4 KB records).

Printed: one JSON line with resolved selections/s (the headline), miss-fetch
GB/s against host-link peaks measured in the same run, the dominant kernel's
roofline (the fetch kernel, bound by the host link), a hit-only leg for the
metadata path against a measured HBM peak, the MLA attention consumer at the
latent-record shape, a sweep of every workload's throughput and link
fraction against the same run's peaks, and the CPU oracle timed on a bounded
sample of the same workload (one pinned core, then every core).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PCIE5_X16_GBPS = 63.0  # 32 GT/s x 16 lanes, 128b/130b line code, per direction
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published


def fetch_traffic(workload="mla_latent"):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per fetch_kernel launch of a
    workload from its committed counter summary, or None if there is none or
    the kernel source changed since it was taken."""
    return counter_traffic(os.path.join("profiles", f"fetch_kernel_traffic_{workload}.md"), "fetch.hip")


def attention_traffic():
    """Scaled FETCH_SIZE + WRITE_SIZE bytes of one MLA attention call (partial
    and combine kernels) at 16 requests x 128 heads x k = 2048, from the
    committed counter summary, or None if the kernels' source changed since."""
    return counter_traffic(os.path.join("profiles", "mla_attention_mla_latent.md"), "attend.hip")


def counter_traffic(rel, source):
    """The `| read (scaled FETCH_SIZE) | N |` and `| written (scaled
    WRITE_SIZE) | N |` rows of a counter summary, if the summary names the
    current sha256 prefix of the measured source file."""
    import hashlib
    import re
    prof = os.path.join(ROOT, rel)
    src = os.path.join(ROOT, "hierarchical_kv_cache_resolve_amd", "csrc", source)
    try:
        text = open(prof).read()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    m = re.search(r"sha256 prefix ([0-9a-f]{16})", text)
    rd = re.search(r"\| read \(scaled FETCH_SIZE\) \| (\d+) \|", text)
    wr = re.search(r"\| written \(scaled WRITE_SIZE\) \| (\d+) \|", text)
    if not (m and rd and wr) or m.group(1) != digest:
        return None
    return {"read_bytes": int(rd.group(1)), "write_bytes": int(wr.group(1)),
            "total_bytes": int(rd.group(1)) + int(wr.group(1)), "source": rel}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="gqa_record")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-hit-only", action="store_true")
    ap.add_argument("--no-probes", action="store_true")
    ap.add_argument("--markers", action="store_true",
                    help="roctx ranges around each timed step (eager steps with --graph 0, else the graph) and "
                         "every library call that enqueues work (rocprofv3 --marker-trace)")
    ap.add_argument("--probe", default="default", choices=["default", "page_table", "slot_scan", "slot_scan_hash"],
                    help="how the metadata kernel finds hits (default: the library's)")
    ap.add_argument("--meta-lanes", type=int, default=0, choices=[0, 512, 1024],
                    help="lanes a (request, layer) of the metadata kernel (0: the library's choice)")
    ap.add_argument("--meta-wgs", type=int, default=None,
                    help="workgroups per (request, layer) that plan alike and copy their misses (0: a separate "
                         "fetch launch, -1: by launch size; default: the library's)")
    ap.add_argument("--fetch-blocks", type=int, default=0)
    ap.add_argument("--prefetch-blocks", type=int, default=None,
                    help="workgroups of the prefetch's side-stream copy launch (default: the library's)")
    ap.add_argument("--unroll", type=int, default=0)
    ap.add_argument("--coherent", action="store_true")
    ap.add_argument("--timing", type=int, default=1, help="replay the timed steps with HIP events on every launch")
    ap.add_argument("--graph", type=int, default=1, help="run the timed steps as one captured HIP graph")
    ap.add_argument("--prefetch", type=int, default=1, help="shared-selection workloads: replay anchor plans")
    ap.add_argument("--consumer", default="auto", choices=["auto", "none", "checksum", "attention"],
                    help="kernel run after every layer's RESOLVE inside the timed steps (auto: shared-selection "
                         "workloads get MLA attention when the records are 576-element bf16 latents, else the "
                         "gather checksum; other workloads none)")
    ap.add_argument("--heads", type=int, default=128, help="query heads of the MLA attention consumer")
    ap.add_argument("--attn-heads-per-wg", type=int, default=0, choices=[0, 32, 64],
                    help="heads per attention workgroup (0: the library chooses by shape)")
    ap.add_argument("--no-attention-leg", action="store_true",
                    help="skip the separate timing of the MLA attention consumer on the workload's shape")
    ap.add_argument("--hit-only-workload", default="gqa_record",
                    help="shapes of the hit-only leg (its pool aliases every history onto one region)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the sweep of the other workloads (each on an aliased 4 GiB pool)")
    ap.add_argument("--sweep-steps", type=int, default=24)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the RESOLVE path shards by "
              "(request, layer) with no exchange, and this benchmark measures one GPU's share.", flush=True)
        sys.exit(2)
    import torch

    import hierarchical_kv_cache_resolve_amd as hs
    import tracegen as tg

    w = tg.WORKLOADS[args.workload]
    mla_records = w.W_KV == 576 and w.elem_bytes == 2
    if args.consumer == "auto":
        args.consumer = ("attention" if mla_records else "checksum") if w.group > 1 else "none"
    if args.consumer == "attention" and not mla_records:
        raise SystemExit("the attention consumer needs 576-element bf16 records")
    W, K = args.warmup, args.steps
    nthreads = max(1, min(16, os.cpu_count() or 1))
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    log(f"workload {w.name}: R={w.num_req} layers={w.num_layers} L_ctx={w.L_ctx} k={w.k} B={w.B} "
        f"row={w.row_bytes}B steps W={W} K={K}")
    t0 = time.time()
    tr = tg.trace(w, steps=W + K, threads=nthreads)
    log(f"trace {tr.nbytes / 1e6:.0f} MB in {time.time() - t0:.1f}s")
    t0 = time.time()
    pool = hs.HostPool.allocate(w.pool_rows * w.row_bytes, coherent=args.coherent)
    tg.pool_fill(pool.ptr, 0, w.pool_rows * w.W_KV, w.pool_seed, nthreads)
    log(f"pool {pool.nbytes / 1e9:.1f} GB pinned+filled in {time.time() - t0:.1f}s")

    res = hs.Resolver(w.num_req, w.num_layers, w.B, w.W_KV, hs.BF16, pool, w.L_ctx, w.pool_rows,
                      region_row=w.region_rows())
    if args.probe != "default":
        res.set_option(hs.HS_OPT_PROBE, {"page_table": hs.HS_PROBE_PAGE_TABLE, "slot_scan": hs.HS_PROBE_SLOT_SCAN,
                                         "slot_scan_hash": hs.HS_PROBE_SLOT_SCAN_HASH}[args.probe])
    if args.attn_heads_per_wg:
        res.set_option(hs.HS_OPT_ATTN_HEADS, args.attn_heads_per_wg)
    if args.fetch_blocks:
        res.set_option(hs.HS_OPT_FETCH_BLOCKS, args.fetch_blocks)
    if args.prefetch_blocks is not None:
        res.set_option(hs.HS_OPT_PREFETCH_BLOCKS, args.prefetch_blocks)
    if args.meta_lanes:
        res.set_option(hs.HS_OPT_META_LANES, args.meta_lanes)
    if args.meta_wgs is not None:
        res.set_option(hs.HS_OPT_META_WGS, args.meta_wgs)
    if args.markers:
        res.set_option(hs.HS_OPT_MARKERS, 1)
    if args.unroll:
        res.set_option(hs.HS_OPT_FETCH_UNROLL, args.unroll)
    sel = torch.from_numpy(tr).to(dev)
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    use_prefetch = w.group > 1 and args.prefetch
    side = torch.cuda.Stream() if use_prefetch else None
    cs = torch.empty((w.num_layers, w.num_req), dtype=torch.int64, device=dev) if args.consumer == "checksum" else None
    attn = None
    if args.consumer == "attention":
        attn = attention_buffers(torch, w, args.heads, dev)
        res.attend_mla(0, attn["q"], out[0], attn["scale"], attn["o"], attn["lse"])   # sizes the workspace
        torch.cuda.synchronize()

    def consume(l, sp):
        if cs is not None:
            res.gather_checksum(l, out[l], cs[l], sp)
        elif attn is not None:
            res.attend_mla(l, attn["q"], out[l], attn["scale"], attn["o"], attn["lse"], sp)

    step = make_step(res, w, sel, out, consume, side, use_prefetch)

    mark = roctx_ranges(args.markers)

    def timed_run(prefetch):
        """Run steps W..W+K-1 (as one captured graph unless --graph 0); returns seconds."""
        if args.graph:
            # the timed steps as one HIP graph: every input already resident,
            # every pointer fixed, the step clock on the device
            with mark(f"timed steps {W}..{W + K - 1} (one graph)"):
                return graph_time(torch, step, W, W + K, prefetch)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(W, W + K):
            with mark(f"step {t}"):
                step(t, sptr, prefetch=prefetch)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    for t in range(W):
        step(t, sptr)
    torch.cuda.synchronize()
    s0 = res.stats()
    elapsed = timed_run(use_prefetch)
    s1 = res.stats()
    code, el, er = res.error()
    if code:
        raise SystemExit(f"device error {code} at layer {el} request {er}")

    # Per-kernel durations: HIP events around every launch perturb the step
    # (about 1 us per event), so they are taken on a replay of the same steps
    # from a reset cache, not on the headline run above.
    tim = None
    if args.timing:
        res.reset()
        for t in range(W):
            step(t, sptr)
        res.set_option(hs.HS_OPT_TIMING, 1)
        res.timing(clear=True)
        r0 = res.stats()
        anchors = set(range(0, w.num_layers, w.group)) if use_prefetch else set()
        r0_layers = [res.stats(l) if l in anchors else None for l in range(w.num_layers)]
        for t in range(W, W + K):
            step(t, sptr)
        torch.cuda.synchronize()
        r1 = res.stats()
        r1_layers = [res.stats(l) if l in anchors else None for l in range(w.num_layers)]
        tim = res.timing(clear=True)
        res.set_option(hs.HS_OPT_TIMING, 0)
        if r1.miss_bytes - r0.miss_bytes != s1.miss_bytes - s0.miss_bytes:
            raise SystemExit("instrumented replay moved different bytes than the timed run")

    prefetch_cmp = None
    if use_prefetch:
        res.reset()
        for t in range(W):
            step(t, sptr, prefetch=False)
        off = timed_run(False)
        prefetch_cmp = {"workload": w.name, "ms_per_step_prefetch_on": elapsed * 1e3 / K, "ms_per_step_prefetch_off": off * 1e3 / K,
                        "consumer_between_layers": args.consumer,
                        "saving": 1.0 - elapsed / off}
        log(f"prefetch on {elapsed * 1e3 / K:.3f} ms/step, off {off * 1e3 / K:.3f} ms/step")
        prefetch_cmp.update(exposed_io(hs, torch, res, w, step, W, K, sptr))

    sels = K * w.num_layers * w.num_req * w.k
    misses = s1.misses - s0.misses
    miss_bytes = s1.miss_bytes - s0.miss_bytes
    value = sels / elapsed
    ms_per_step = elapsed * 1e3 / K
    log(f"timed: {ms_per_step:.3f} ms/step, {value / 1e6:.1f} M sel/s, miss rate {misses / sels:.4f}, "
        f"miss {miss_bytes / elapsed / 1e9:.2f} GB/s")

    result = {
        "metric": "resolved selections/s per layer-step + miss-fetch GB/s vs measured host-link peak",
        "value": value,
        "unit": "selections/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic (seeded selection trace and N(0,1) bf16 host pool)",
        "config": {"workload": f"{w.name}: {w.num_req} requests x {w.num_layers} layers, L_ctx={w.L_ctx}, "
                               f"W_KV={w.W_KV} bf16 ({w.row_bytes} B records), k={w.k}, B={w.B}, "
                               f"retention {w.p_keep}, +-{w.window} locality window",
                   "num_req": w.num_req, "num_layers": w.num_layers, "L_ctx": w.L_ctx, "k": w.k, "B": w.B,
                   "record_bytes": w.row_bytes, "host_pool_GB": round(pool.nbytes / 1e9, 2),
                   "probe": "slot_scan" if args.probe == "default" else args.probe,
                   "parallelism": "single GPU"},
        "miss_rate": misses / sels,
        "miss_fetch_GBps": miss_bytes / elapsed / 1e9,
        "selections_per_layer_step": w.num_req * w.k,
        "layer_steps_per_s": K * w.num_layers / elapsed,
    }
    if prefetch_cmp:
        result["prefetch"] = prefetch_cmp

    # peaks measured in the same run
    link_sdma = link_kernel = hbm_peak = None
    if not args.no_probes:
        nb = 1 << 30
        hp = hs.hisparse_host_alloc(nb, args.coherent)
        try:
            d = torch.empty(nb, dtype=torch.uint8, device=dev)
            link_sdma = hs.hisparse_probe_link_sdma(hp, d.data_ptr(), nb, 5, sptr)
            link_kernel = hs.hisparse_probe_link_kernel(hp, d.data_ptr(), nb, 5, sptr)
            del d
        finally:
            hs.hisparse_host_free(hp)
        nb = 4 << 30
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        hbm_peak = hs.hisparse_probe_hbm(a.data_ptr(), b.data_ptr(), nb, 5, sptr)
        del a, b
        torch.cuda.synchronize()
        log(f"peaks: link sdma {link_sdma:.1f} GB/s, link kernel {link_kernel:.1f} GB/s, hbm copy {hbm_peak:.0f} GB/s")
    link_peak = max(x for x in (link_sdma, link_kernel, 1e-9) if x is not None)
    result["link_peak_GBps"] = {"sdma_copy": link_sdma, "kernel_16B_loads": link_kernel,
                                "published_pcie5_x16": PCIE5_X16_GBPS}
    result["miss_fetch_frac_of_link_peak"] = result["miss_fetch_GBps"] / link_peak if link_sdma else None

    if tim is not None and (tim.fetch_launches or tim.plan_launches):
        # units split over several workgroups copy their misses inside the
        # metadata launch: then that launch is the copying kernel
        split = tim.fetch_launches == 0
        copy_ms, copy_launches = (tim.plan_ms, tim.plan_launches) if split else (tim.fetch_ms, tim.fetch_launches)
        fetch_avg_ms = copy_ms / copy_launches
        plan_avg_ms = tim.plan_ms / tim.plan_launches
        # algorithmic bytes of the fetch kernel: every missed record crosses the
        # host link once (and is written once to HBM).  With prefetch, the main
        # stream's fetch launches carry the anchors' misses only; the shared
        # layers' copies are the replay launches on the side stream.
        if use_prefetch:
            fetch_bytes = sum(r1l.miss_bytes - r0l.miss_bytes for r0l, r1l in zip(r0_layers, r1_layers)
                              if r0l is not None)
        else:
            fetch_bytes = miss_bytes
        achieved = fetch_bytes / (copy_ms * 1e-3) / 1e9
        result["roofline"] = {
            "kernel": ("bitmap_resolve_kernel (units split over workgroups: plan and host-mapped 16 B loads -> HBM "
                       "cache rows in one launch)" if split else
                       "fetch_kernel (host-mapped 16 B loads -> HBM cache rows)"),
            "bound": "host_link",
            "achieved": achieved,
            "peak": link_peak,
            "unit": "GB/s",
            "frac": achieved / link_peak,
            "frac_published": achieved / PCIE5_X16_GBPS,
            # HBM + link bytes of the workload's fetch launches from its committed counter summary
            # (None if there is none, or if the kernel source changed since it was taken)
            "traffic": None if split else (fetch_traffic(w.name) or {}).get("total_bytes"),
            "traffic_detail": None if split else fetch_traffic(w.name),
            "peak_note": "peak = max(SDMA H2D copy, 16 B-load streaming kernel) measured in this run; "
                         f"frac_published against PCIe 5.0 x16 = {PCIE5_X16_GBPS} GB/s per direction",
            "avg_launch_ms": fetch_avg_ms,
            "bytes_per_launch": fetch_bytes / copy_launches,
        }
        if tim.replay_launches:
            result["kernels_replay"] = {"replay_avg_ms": tim.replay_ms / tim.replay_launches,
                                        "replay_launches": tim.replay_launches,
                                        "publish_avg_ms": tim.publish_ms / max(1, tim.publish_launches),
                                        "replay_GBps": (miss_bytes - fetch_bytes) / (tim.replay_ms * 1e-3) / 1e9}
        result["kernels"] = {
            "split_units": split,
            "fetch_avg_ms": fetch_avg_ms if not split else None, "fetch_launches": tim.fetch_launches,
            "plan_avg_ms": plan_avg_ms, "plan_launches": tim.plan_launches,
            "plan_share_of_step": tim.plan_ms / (elapsed * 1e3),
            "fetch_share_of_step": copy_ms / (elapsed * 1e3),
            "timing_dropped": tim.dropped,
        }
        log(f"{'split resolve' if split else 'fetch'} avg {fetch_avg_ms * 1e3:.1f} us ({achieved:.1f} GB/s), "
            f"plan avg {plan_avg_ms * 1e3:.1f} us")

    if not args.no_attention_leg and mla_records:
        result["attention"] = attention_leg(hs, torch, res, w, out, args.heads, dev, hbm_peak,
                                            heads_per_wg=args.attn_heads_per_wg)

    res.close()

    if not args.no_attention_leg and not mla_records:
        # the consumer needs 576-element latent records: it runs at the latent
        # workload's shape on a pool that aliases every history onto one region
        result["attention"] = attention_leg_latent_shape(hs, tg, torch, dev, sptr, args.heads, hbm_peak,
                                                         heads_per_wg=args.attn_heads_per_wg)

    if not args.no_hit_only:
        result["hit_only"] = hit_only_leg(hs, tg, torch, tg.WORKLOADS[args.hit_only_workload], dev, sptr, hbm_peak,
                                          meta_lanes=args.meta_lanes, meta_wgs=args.meta_wgs)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(tg, w, tr, pool, W, args.cpu_seconds)
        result["cpu_baseline_threads"] = cpu_baseline_threads(tg, w, tr, pool, W,
                                                              result["cpu_baseline"]["steps"])

    # the pinned pools of the sweep fit only once the workload's pool is released
    pool.free()
    if not args.no_sweep:
        result["sweep"] = sweep(hs, tg, torch, dev, sptr, w.name, link_peak if link_sdma else None,
                                args.sweep_steps, nthreads, args.heads)
        if "prefetch" not in result:
            for row in result["sweep"].values():
                if "prefetch" in row:
                    result["prefetch"] = row["prefetch"]
    print(json.dumps(result), flush=True)


def roctx_ranges(on):
    """A context manager factory: with `on`, each `with mark(name)` is one roctx
    range (the profiler's marker library, recorded by rocprofv3
    --marker-trace); otherwise it does nothing."""
    import contextlib
    import ctypes
    lib = None
    if on:
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            try:
                lib = ctypes.CDLL(name)
                break
            except OSError:
                pass
        if lib is None:
            raise SystemExit("--markers: the roctx library (librocprofiler-sdk-roctx) cannot be loaded")
        lib.roctxRangePushA.argtypes = [ctypes.c_char_p]

    @contextlib.contextmanager
    def mark(name):
        if lib is not None:
            lib.roctxRangePushA(name.encode())
        try:
            yield
        finally:
            if lib is not None:
                lib.roctxRangePop()
    return mark


def make_step(res, w, sel, out, consume, side, default_prefetch):
    """One decode step of the workload: RESOLVE of every layer, each followed
    by the consumer.  With exact prefetch (shared-selection groups), each
    anchor is resolved, its plan replayed into the group's shared layers on
    the side stream, and the shared layers then only publish.  `hook(l,
    when)` runs right before and after each shared layer's resolve."""
    import torch

    def step(t, sp, capturing=False, prefetch=None, hook=None):
        if prefetch is None:
            prefetch = default_prefetch
        if not prefetch:
            for l in range(w.num_layers):
                if hook:
                    hook(l, "before")
                res.resolve(l, sel[t, l], out[l], sp)
                if hook:
                    hook(l, "after")
                consume(l, sp)
            return
        for g0 in range(0, w.num_layers, w.group):
            res.resolve(g0, sel[t, g0], out[g0], sp)
            shared = list(range(g0 + 1, min(g0 + w.group, w.num_layers)))
            if capturing:
                side.wait_stream(torch.cuda.current_stream())
            res.prefetch(g0, shared, side)
            consume(g0, sp)
            for l in shared:
                if hook:
                    hook(l, "before")
                res.resolve(l, sel[t, l], out[l], sp)
                if hook:
                    hook(l, "after")
                consume(l, sp)

    return step


def graph_time(torch, step, t0, t1, prefetch):
    """Capture steps t0..t1-1 as one HIP graph, replay it once; seconds."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream().cuda_stream
        for t in range(t0, t1):
            step(t, cap, capturing=True, prefetch=prefetch)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t_start
    del graph
    return dt


def attention_buffers(torch, w, heads, dev):
    """Query, output and log-sum-exp buffers of the MLA decode consumer: seeded
    N(0,1) queries in bf16, one per head, in the 576-element record space."""
    g = torch.Generator(device="cpu").manual_seed(260807)
    q = torch.randn((w.num_req, heads, 576), generator=g).to(torch.bfloat16).to(dev).view(torch.int16)
    return {"q": q, "scale": 1.0 / 24.0,
            "o": torch.empty((w.num_req, heads, 512), dtype=torch.float32, device=dev),
            "lse": torch.empty((w.num_req, heads), dtype=torch.float32, device=dev)}


def attention_leg(hs, torch, res, w, out, heads, dev, hbm_peak, iters=20, heads_per_wg=0, warm=20):
    """The consumer alone: sparse MLA decode attention over the slots the last
    timed step published, every layer, timed with HIP events on the stream
    the kernels run on, after `warm` untimed passes over the layers (the
    leg follows link-bound work, and the first few milliseconds of attention
    after it run slower).  Algorithmic work per (request, layer): k records
    of 1152 B read once, heads x k x (576 + 512) multiply-adds."""
    a = attention_buffers(torch, w, heads, dev)
    for _ in range(warm):
        for l in range(w.num_layers):
            res.attend_mla(l, a["q"], out[l], a["scale"], a["o"], a["lse"])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        for l in range(w.num_layers):
            res.attend_mla(l, a["q"], out[l], a["scale"], a["o"], a["lse"])
    e1.record()
    torch.cuda.synchronize()
    res.check_error()
    us = e0.elapsed_time(e1) * 1e3 / (iters * w.num_layers)
    flops = 2.0 * w.num_req * heads * w.k * (576 + 512)
    rec_bytes = w.num_req * w.k * w.row_bytes
    io_bytes = rec_bytes + w.num_req * heads * (576 * 2 + 512 * 4 + 4) + w.num_req * w.k * 4
    tflops = flops / (us * 1e-6) / 1e12
    gbps = io_bytes / (us * 1e-6) / 1e9
    log(f"attention: {us:.1f} us per layer ({tflops:.0f} TFLOP/s, {gbps:.0f} GB/s of records+q+out)")
    # counter traffic is summarised for the benchmark's own shape only
    tr = (attention_traffic() if (w.num_req, heads, w.k, w.row_bytes, heads_per_wg) == (16, 128, 2048, 1152, 0)
          else None)
    if tr:
        tr["over_algorithmic"] = tr["total_bytes"] / io_bytes
    return {"kernels": "mla_partial_kernel + mla_combine_kernel", "heads": heads, "k": w.k,
            "heads_per_workgroup": heads_per_wg or "by shape",
            "requests": w.num_req, "us_per_layer": us, "TFLOPs": tflops,
            "mfma_frac": tflops / MFMA_BF16_TFLOPS, "algorithmic_GBps": gbps,
            "hbm_frac_published": gbps / HBM_PEAK_GBPS,
            "hbm_frac_measured_copy": gbps / hbm_peak if hbm_peak else None,
            "algorithmic_bytes": io_bytes, "flops": flops, "traffic": tr}


def hit_only_leg(hs, tg, torch, w, dev, sptr, hbm_peak, steps=64, meta_lanes=0, meta_wgs=None):
    """Metadata path alone: every step after the first repeats it, so every
    selection hits and nothing crosses the host link.  Timed as captured HIP
    graphs (one per variant) so that host launch cost does not enter.  Only
    the first (filling) step reads the pool, so every history aliases onto
    one region of L_ctx rows."""
    wh = tg.hit_only(w)
    tr = torch.from_numpy(tg.trace(wh, steps=2)).to(dev)
    pool = hs.HostPool.allocate(w.L_ctx * w.row_bytes)
    tg.pool_fill(pool.ptr, 0, w.L_ctx * w.W_KV, w.pool_seed)
    res = hs.Resolver(w.num_req, w.num_layers, w.B, w.W_KV, hs.BF16, pool, w.L_ctx, w.L_ctx,
                      region_row=np.zeros(w.num_req * w.num_layers, dtype=np.int64))
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    if meta_lanes:
        res.set_option(hs.HS_OPT_META_LANES, meta_lanes)
    if meta_wgs is not None:
        res.set_option(hs.HS_OPT_META_WGS, meta_wgs)
    for l in range(w.num_layers):
        res.resolve(l, tr[0, l], out[l], sptr)
    # algorithmic bytes per (request, layer) of an all-hit resolve with the
    # slot scan (the default probe): read the selection (4k) and the slot map
    # (4B); write the hit stamps (4k) and the published slots (4k).  The
    # page-table probe also reads the k page-table entries the selection names.
    per_rl = 4 * w.k + 4 * w.B + 4 * w.k + 4 * w.k
    per_rl_pt = per_rl + 4 * w.k
    layers = list(range(w.num_layers))
    nb = max(1, min(len(layers), 8192 // w.num_req, 32))  # layers per batched launch
    batches = [layers[i:i + nb] for i in range(0, len(layers), nb)]
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            for l in layers:
                res.resolve(l, tr[1, l], out[l], cap)
    with torch.cuda.graph(g2):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            for b in batches:
                res.resolve_layers(b, [tr[1, l] for l in b], [out[l] for l in b], cap)
    torch.cuda.synchronize()
    g1.replay()  # warm
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g1.replay()
    torch.cuda.synchronize()
    per_layer = time.perf_counter() - t0
    t0 = time.perf_counter()
    g2.replay()
    torch.cuda.synchronize()
    batched = time.perf_counter() - t0
    # the same batched launches with the page-table probe (one page-table load
    # per selected position instead of the slot scan)
    res.set_option(hs.HS_OPT_PROBE, hs.HS_PROBE_PAGE_TABLE)
    g3 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g3):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            for b in batches:
                res.resolve_layers(b, [tr[1, l] for l in b], [out[l] for l in b], cap)
    torch.cuda.synchronize()
    g3.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g3.replay()
    torch.cuda.synchronize()
    batched_pt = time.perf_counter() - t0
    res.set_option(hs.HS_OPT_PROBE, hs.HS_PROBE_SLOT_SCAN)
    # the per-layer launches with each (request, layer) split over several
    # workgroups that plan it alike and would copy its misses themselves: one
    # launch a layer (the default keeps the fetch launch at shapes whose
    # misses could reach tens of MB)
    split_g = max(1, min(32, -(-256 // w.num_req)))
    res.set_option(hs.HS_OPT_META_WGS, split_g)
    g4 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g4):
        cap = torch.cuda.current_stream().cuda_stream
        for _ in range(steps):
            for l in layers:
                res.resolve(l, tr[1, l], out[l], cap)
    torch.cuda.synchronize()
    g4.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g4.replay()
    torch.cuda.synchronize()
    per_layer_split = time.perf_counter() - t0
    res.set_option(hs.HS_OPT_META_WGS, -1 if meta_wgs is None else meta_wgs)
    st = res.stats()
    del g1, g2, g3, g4
    res.close()
    pool.free()
    total = per_rl * w.num_req * w.num_layers * steps
    total_pt = per_rl_pt * w.num_req * w.num_layers * steps
    r = {
        "workload": f"{w.name} shapes: {w.num_req} requests x {w.num_layers} layers, k={w.k}, B={w.B}",
        "bytes_per_request_layer": per_rl,
        "bytes_per_request_layer_page_table_probe": per_rl_pt,
        "per_layer_launch_GBps": total / per_layer / 1e9,
        "per_layer_resolve_us": per_layer / (steps * w.num_layers) * 1e6,
        "per_layer_split_resolve_us": per_layer_split / (steps * w.num_layers) * 1e6,
        "per_layer_split_wgs": split_g,
        "batched_all_layers_GBps": total / batched / 1e9,
        "batched_step_us": batched / steps * 1e6,
        "batched_page_table_GBps": total_pt / batched_pt / 1e9,
        "batched_page_table_step_us": batched_pt / steps * 1e6,
        "batched_launches_per_step": len(batches),
        "hbm_peak_GBps": hbm_peak,
        "hbm_published_GBps": 8000.0,
        "misses_after_fill": int(st.misses - w.num_req * w.num_layers * w.k),
        "timing": "wall clock around one replay of a captured graph",
    }
    if hbm_peak:
        r["per_layer_frac_of_hbm_peak"] = r["per_layer_launch_GBps"] / hbm_peak
        r["per_layer_split_frac_of_hbm_peak"] = total / per_layer_split / 1e9 / hbm_peak
        r["batched_frac_of_hbm_peak"] = r["batched_all_layers_GBps"] / hbm_peak
        r["batched_page_table_frac_of_hbm_peak"] = r["batched_page_table_GBps"] / hbm_peak
    log(f"hit-only: per-layer {r['per_layer_resolve_us']:.1f} us/resolve ({r['per_layer_launch_GBps']:.1f} GB/s; "
        f"split units {r['per_layer_split_resolve_us']:.1f} us), "
        f"batched {r['batched_step_us']:.1f} us/step ({r['batched_all_layers_GBps']:.1f} GB/s), "
        f"batched page-table probe {r['batched_page_table_step_us']:.1f} us/step "
        f"({r['batched_page_table_GBps']:.1f} GB/s)")
    return r


def exposed_io(hs, torch, res, w, step, W, K, sptr):
    """Exact prefetch on a shared-selection workload: how much of the shared
    layers' resolve time the main stream still waits for.  The same K steps
    run twice from a reset cache, prefetch off and on, with HIP events on the
    main stream right before and after every shared layer's resolve; with
    prefetch off that interval is the layer's own metadata work and host
    fetch, with prefetch on it is the wait for the side stream's replay plus
    the publish-only resolve.  The replay's own duration on the side stream
    comes from the library's per-launch timing."""
    shared = [l for l in range(w.num_layers) if l % w.group != 0]
    out = {}
    for prefetch in (False, True):
        res.reset()
        for t in range(W):
            step(t, sptr, prefetch=prefetch)
        torch.cuda.synchronize()
        ev = []
        res.set_option(hs.HS_OPT_TIMING, 1)
        res.timing(clear=True)

        def hook(l, when, _ev=ev):
            if l in shared:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                _ev.append((l, when, e))

        for t in range(W, W + K):
            step(t, sptr, prefetch=prefetch, hook=hook)
        torch.cuda.synchronize()
        tim = res.timing(clear=True)
        res.set_option(hs.HS_OPT_TIMING, 0)
        total = 0.0
        for (l0, w0, e0), (l1, w1, e1) in zip(ev[0::2], ev[1::2]):
            assert l0 == l1 and w0 == "before" and w1 == "after"
            total += e0.elapsed_time(e1)
        key = "on" if prefetch else "off"
        out[f"exposed_io_ms_{key}"] = total / K
        if prefetch:
            out["replay_ms_per_step"] = tim.replay_ms / K
            out["replay_launches_per_step"] = tim.replay_launches / K
    out["io_hidden_frac"] = 1.0 - out["exposed_io_ms_on"] / out["exposed_io_ms_off"]
    out["shared_layers"] = shared
    out["exposed_io_note"] = ("per step, summed over the shared layers: main-stream time from right before to "
                              "right after each shared layer's resolve (HIP events on the main stream)")
    log(f"exposed shared-layer resolve: off {out['exposed_io_ms_off']:.3f} ms/step, "
        f"on {out['exposed_io_ms_on']:.3f} ms/step -> hidden {out['io_hidden_frac']:.2f}")
    return out


def prefetch_leg(hs, torch, res, w, sel, out, dev, sptr, W, K, heads):
    """Exact prefetch on a shared-selection workload with MLA attention after
    every layer: the step time with prefetch on and off (one captured graph
    each, from a reset cache after W warm steps), then the shared layers'
    exposed resolve time both ways (exposed_io)."""
    side = torch.cuda.Stream()
    attn = attention_buffers(torch, w, heads, dev)
    res.attend_mla(0, attn["q"], out[0], attn["scale"], attn["o"], attn["lse"])  # sizes the workspace
    torch.cuda.synchronize()

    def consume(l, sp):
        res.attend_mla(l, attn["q"], out[l], attn["scale"], attn["o"], attn["lse"], sp)

    step = make_step(res, w, sel, out, consume, side, True)
    secs = {}
    for prefetch in (True, False):
        res.reset()
        for t in range(W):
            step(t, sptr, prefetch=prefetch)
        torch.cuda.synchronize()
        secs[prefetch] = graph_time(torch, step, W, W + K, prefetch)
    r = {"workload": w.name, "consumer_between_layers": "attention",
         "ms_per_step_prefetch_on": secs[True] * 1e3 / K, "ms_per_step_prefetch_off": secs[False] * 1e3 / K,
         "saving": 1.0 - secs[True] / secs[False]}
    log(f"prefetch ({w.name}): on {r['ms_per_step_prefetch_on']:.3f} ms/step, off {r['ms_per_step_prefetch_off']:.3f}")
    r.update(exposed_io(hs, torch, res, w, step, W, K, sptr))
    res.check_error()
    return r


def aliased(w, gib=4):
    """The workload with its pool capped at about `gib` GiB (whole histories;
    histories alias onto the physical regions modulo their number)."""
    rows = max(w.L_ctx, ((gib << 30) // w.row_bytes) // w.L_ctx * w.L_ctx)
    return w.replace(pool_rows_cap=min(rows, w.logical_rows))


def attention_leg_latent_shape(hs, tg, torch, dev, sptr, heads, hbm_peak, heads_per_wg=0):
    """The MLA consumer at the latent-record workload's shape (16 requests,
    k = 2048, 576-element bf16 records, 128 heads), on slots published by two
    RESOLVE steps of that workload over a pool in which every history aliases
    onto one region."""
    w = tg.WORKLOADS["mla_latent"].replace(pool_rows_cap=tg.WORKLOADS["mla_latent"].L_ctx)
    tr = torch.from_numpy(tg.trace(w, steps=2)).to(dev)
    pool = hs.HostPool.allocate(w.pool_rows * w.row_bytes)
    tg.pool_fill(pool.ptr, 0, w.pool_rows * w.W_KV, w.pool_seed)
    res = hs.Resolver(w.num_req, w.num_layers, w.B, w.W_KV, hs.BF16, pool, w.L_ctx, w.pool_rows,
                      region_row=w.region_rows())
    if heads_per_wg:
        res.set_option(hs.HS_OPT_ATTN_HEADS, heads_per_wg)
    out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)
    for t in range(2):
        for l in range(w.num_layers):
            res.resolve(l, tr[t, l], out[l], sptr)
    torch.cuda.synchronize()
    r = attention_leg(hs, torch, res, w, out, heads, dev, hbm_peak, heads_per_wg=heads_per_wg)
    r["workload"] = "mla_latent shapes (16 requests x 8 layers, k=2048, 576-element bf16 records), aliased pool"
    res.close()
    pool.free()
    return r


def sweep(hs, tg, torch, dev, sptr, skip, link_peak, steps, nthreads, heads=128):
    """Every other workload at its full cache shape on an aliased pool of
    about 4 GiB (the host fetch reads whatever row a history's position maps
    to, so only the pool's footprint changes): steps run as one captured
    graph after 8 eager warm-up steps, then replayed with per-launch timing.
    Reports selections/s, the miss fetch over the step and the fetch kernel's
    rate, each against the host-link peak measured earlier in this run.  A
    shared-selection workload with latent records also runs the exact-prefetch
    leg (prefetch on and off, MLA attention between layers, exposed IO)."""
    rows = {}
    warm = 8
    for name, w0 in tg.WORKLOADS.items():
        if name == skip:
            continue
        w = aliased(w0)
        tr = torch.from_numpy(tg.trace(w, steps=warm + steps, threads=nthreads)).to(dev)
        pool = hs.HostPool.allocate(w.pool_rows * w.row_bytes)
        tg.pool_fill(pool.ptr, 0, w.pool_rows * w.W_KV, w.pool_seed, nthreads)
        res = hs.Resolver(w.num_req, w.num_layers, w.B, w.W_KV, hs.BF16, pool, w.L_ctx, w.pool_rows,
                          region_row=w.region_rows())
        out = torch.empty((w.num_layers, w.num_req, w.k), dtype=torch.int32, device=dev)

        def run_steps(t0, t1, sp):
            for t in range(t0, t1):
                for l in range(w.num_layers):
                    res.resolve(l, tr[t, l], out[l], sp)

        run_steps(0, warm, sptr)
        torch.cuda.synchronize()
        s0 = res.stats()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_steps(warm, warm + steps, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        s1 = res.stats()
        del g
        res.reset()
        run_steps(0, warm, sptr)
        res.set_option(hs.HS_OPT_TIMING, 1)
        res.timing(clear=True)
        r0 = res.stats()
        run_steps(warm, warm + steps, sptr)
        torch.cuda.synchronize()
        r1 = res.stats()
        tim = res.timing(clear=True)
        res.set_option(hs.HS_OPT_TIMING, 0)
        res.check_error()
        miss_bytes = s1.miss_bytes - s0.miss_bytes
        sels = steps * w.num_layers * w.num_req * w.k
        split = tim.fetch_launches == 0
        copy_ms = tim.plan_ms if split else tim.fetch_ms
        fetch_gbps = (r1.miss_bytes - r0.miss_bytes) / (copy_ms * 1e-3) / 1e9 if copy_ms else None
        row = {"selections_per_s": sels / dt, "ms_per_step": dt * 1e3 / steps,
               "miss_rate": (s1.misses - s0.misses) / sels, "miss_fetch_GBps": miss_bytes / dt / 1e9,
               "split_units": split,
               "copy_kernel": "bitmap_resolve_kernel (split units)" if split else "fetch_kernel",
               "fetch_kernel_GBps": fetch_gbps, "plan_avg_us": tim.plan_ms * 1e3 / max(1, tim.plan_launches),
               "fetch_avg_us": tim.fetch_ms * 1e3 / max(1, tim.fetch_launches),
               "pool_GB": round(pool.nbytes / 1e9, 2), "logical_pool_GB": round(w.logical_rows * w.row_bytes / 1e9, 1)}
        if link_peak:
            row["miss_fetch_frac_of_link_peak"] = row["miss_fetch_GBps"] / link_peak
            row["fetch_kernel_frac_of_link_peak"] = fetch_gbps / link_peak if fetch_gbps else None
        if w.group > 1 and w.W_KV == 576 and w.elem_bytes == 2:
            row["prefetch"] = prefetch_leg(hs, torch, res, w, tr, out, dev, sptr, warm, steps, heads)
        rows[name] = row
        log(f"sweep {name}: {row['selections_per_s'] / 1e6:.1f} M sel/s, {row['ms_per_step']:.3f} ms/step, "
            f"miss {row['miss_fetch_GBps']:.1f} GB/s, copy kernel "
            f"{fetch_gbps if fetch_gbps else 0:.1f} GB/s, plan {row['plan_avg_us']:.1f} us")
        res.close()
        pool.free()
        del tr, out
        torch.cuda.empty_cache()
    return rows


def gpu_numa_node(torch):
    """NUMA node of the GPU's PCI device (sysfs), or None."""
    try:
        p = torch.cuda.get_device_properties(0)
        bdf = f"{getattr(p, 'pci_domain_id', 0):04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        node = int(open(f"/sys/bus/pci/devices/{bdf}/numa_node").read().strip())
        return node if node >= 0 else None
    except (AttributeError, OSError, ValueError):
        return None


def node_cpus(node):
    """CPUs of a NUMA node that this process may run on (all allowed CPUs if unknown)."""
    allowed = sorted(os.sched_getaffinity(0))
    if node is None:
        return allowed
    try:
        cpus = set()
        for part in open(f"/sys/devices/system/node/node{node}/cpulist").read().strip().split(","):
            lo, _, hi = part.partition("-")
            cpus.update(range(int(lo), int(hi or lo) + 1))
        on_node = [c for c in allowed if c in cpus]
        return on_node or allowed
    except (OSError, ValueError):
        return allowed


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family, model and
    stepping numbers (a virtualised host may give only a short name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                key, val = (x.strip() for x in line.split(":", 1))
                if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                    fields[key] = val
            elif fields:
                break
    except OSError:
        return None
    name = fields.get("model name")
    if name is None:
        return None
    ids = [f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(tg, w, tr, pool, warm_steps, seconds):
    """The oracle as it stands, single-threaded and pinned to one core on the
    GPU's NUMA node, on the first steps of the same workload until about
    `seconds` of resolve time have passed (miss rows copied from the same
    pinned pool into its host cache model).  Runs after every GPU leg."""
    import torch
    from oracle import Oracle
    node = gpu_numa_node(torch)
    core = node_cpus(node)[0]
    saved = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {core})
    try:
        pool_np = pool.numpy_view()
        rr = w.region_rows()
        o = Oracle(w.num_req, w.num_layers, w.B, w.L_ctx, w.row_bytes, model_bytes=True)
        for t in range(warm_steps):
            for l in range(w.num_layers):
                o.resolve(l, tr[t, l], pool_np, rr)
        n_steps, spent = 0, 0.0
        t = warm_steps
        while spent < seconds and t < tr.shape[0]:
            t0 = time.perf_counter()
            for l in range(w.num_layers):
                o.resolve(l, tr[t, l], pool_np, rr)
            spent += time.perf_counter() - t0
            n_steps += 1
            t += 1
        o.close()
    finally:
        os.sched_setaffinity(0, saved)
    sels = n_steps * w.num_layers * w.num_req * w.k
    log(f"cpu oracle (core {core}, node {node}): {n_steps} steps in {spent:.1f}s -> {sels / spent / 1e6:.2f} M sel/s")
    return {"value": sels / spent, "unit": "selections/s", "cores": 1, "kind": "oracle",
            "sample": f"steps {warm_steps}..{warm_steps + n_steps - 1} of {w.name} (all {w.num_req} requests x "
                      f"{w.num_layers} layers, miss rows copied from the same pinned pool), after "
                      f"{warm_steps} untimed warm steps; single thread pinned to one core",
            "steps": n_steps, "core": core, "numa_node": node,
            "numa_note": None if node is not None else
            "the platform reports no NUMA node for the GPU's PCI device (sysfs numa_node -1 or absent): "
            "pinned to the first allowed core",
            "cpu_model": cpu_model()}


def cpu_baseline_threads(tg, w, tr, pool, warm_steps, n_steps):
    """The same oracle sample on every allowed core: the (request, layer)
    units are independent, so each thread owns a share of them (one oracle
    instance per unit) and runs all their steps; each thread is pinned to its
    own core.  Wall clock around the timed steps of all threads."""
    import threading
    from oracle import Oracle
    pool_np = pool.numpy_view()
    rr = w.region_rows()
    cpus = sorted(os.sched_getaffinity(0))
    n = len(cpus)
    units = [(r, l) for r in range(w.num_req) for l in range(w.num_layers)]
    shares = [units[i::n] for i in range(n)]
    ready = threading.Barrier(n + 1)
    go = threading.Barrier(n + 1)
    done = threading.Barrier(n + 1)

    def worker(i):
        os.sched_setaffinity(0, {cpus[i]})
        mine = [(r, l, Oracle(1, 1, w.B, w.L_ctx, w.row_bytes, model_bytes=True),
                 np.array([rr[r * w.num_layers + l]], dtype=np.int64)) for r, l in shares[i]]
        for t in range(warm_steps):
            for r, l, o, reg in mine:
                o.resolve(0, tr[t, l, r:r + 1], pool_np, reg)
        ready.wait()
        go.wait()
        for t in range(warm_steps, warm_steps + n_steps):
            for r, l, o, reg in mine:
                o.resolve(0, tr[t, l, r:r + 1], pool_np, reg)
        done.wait()
        for _, _, o, _ in mine:
            o.close()

    th = [threading.Thread(target=worker, args=(i,)) for i in range(n)]
    for x in th:
        x.start()
    ready.wait()
    t0 = time.perf_counter()
    go.wait()
    done.wait()
    spent = time.perf_counter() - t0
    for x in th:
        x.join()
    sels = n_steps * w.num_layers * w.num_req * w.k
    log(f"cpu oracle, {n} threads: {n_steps} steps in {spent:.2f}s -> {sels / spent / 1e6:.2f} M sel/s")
    return {"value": sels / spent, "unit": "selections/s", "cores": n, "kind": "oracle",
            "sample": f"the single-thread sample, {len(units)} (request, layer) units spread over {n} threads, "
                      "one per allowed core", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "allowed_cpus": n}


if __name__ == "__main__":
    main()

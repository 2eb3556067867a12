"""Benchmark: MoE-stack decode tokens/s through the offloaded MoE layers on one MI355X.

A step is one decode step of the whole stack: for a batch of b tokens, every
one of the L layers runs the router, the LRU plan and miss uploads, the
expert GEMVs and the combine (residual chained, x_{l+1} = x_l + y_l).  Inputs
(AR(1) hidden states, router weights) are resident in HBM before timing; the
expert store is pinned host memory holding every (layer, expert) block.

Protocol per batch size, on a cache that starts empty:
  * cold start: the first steps from the empty cache (64 one-token steps, the
    point where a 256-step trace is taken to be in its steady state; fewer for
    large batches), timed as one window and reported as `cold_start`;
  * --warmup untimed steps;
  * three windows of --steps timed steps each, each bracketed by a device
    synchronisation; `value` is the median window's tokens/s.
Every window is also bracketed, outside its timed region, by a marker kernel
(a one-element bitwise_not), so that `--mode trace-summary` can cut a rocprofv3
kernel trace of the same command down to the timed windows.

Prints one JSON line (the driver's contract) with, in addition, the roofline of
the kernel class with the most GPU time (HIP events recorded by the dispatch
on its launch stream), the all-resident bound, the pinned host-to-device link
rate and the CPU oracle timed on a bounded sample of the workload.
"""
import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-stack decode tokens/s (b=1,4,32) + % HBM peak; cache hit rate"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense fp16/bf16 MFMA, MI355X

WORKLOADS = {
    # Qwen3-30B-A3B-shaped stack (SGLang page, "What does Paged Experts actually do?"): a
    # host store of all 48 x 128 distinct blocks (16.3 GB pinned)
    "qwen3-30b-a3b-int4": dict(L=48, E=128, k=8, H=2048, I=768, quant=1, K=92, pool_shared=False,
                               shared_expert=False, distinct=None, pf_ahead=5),
    # Qwen3.8-Flash-Next-shaped stack, e2m1 + E4M3, shared pool of 2048 slots, shared expert; its
    # 65 GB store is drawn as 1031 distinct blocks mapped onto the 48 x 512 keys
    "qwen3.8-flash-next-e2m1": dict(L=48, E=512, k=10, H=3072, I=512, quant=2, K=2048, pool_shared=True,
                                    shared_expert=True, distinct=1031, pf_ahead=1),
    "tiny-fp32": dict(L=1, E=16, k=2, H=256, I=128, quant=0, K=8, pool_shared=False, shared_expert=False,
                      distinct=None, pf_ahead=3),
}
QUANT_NAME = {0: "f32", 1: "int4_g32_f16", 2: "e2m1_g16_e4m3"}
DTYPE = {0: "f32", 1: "int4xf16", 2: "e2m1xf16"}

# kernel classes the library times, with the kernels each stands for
KERNEL_NAME = {
    "router": "k_router_fused / k_router_logits + k_router_select (float64 logits, softmax, top-k; this layer's "
              "router and the speculative ones)",
    "gate_up_early": "k_expert_gemv_pre (one-token gate/up + SwiGLU of the resident picks, launched before the plan)",
    "gate_up": "k_expert_gemv / k_expert_gemv_stream gate/up (SwiGLU) GEMV",
    "down": "k_down_combine (down projection + weighted combine) / k_expert_gemv down",
    "expert_fused": "k_expert_fused (gate/up + SwiGLU, down + combine, one launch)",
    "down_early": "k_down_combine_picks (one-token down + combine of the resident picks, launched before the plan; "
                  "in captured steps the layer's down)",
}
KERNEL_SOURCES = {"router": ("expert_offload_lru_amd/csrc/router.hip", "expert_offload_lru_amd/csrc/kernels.hpp")}
GEMV_SOURCES = ("expert_offload_lru_amd/csrc/expert_gemv.hip", "expert_offload_lru_amd/csrc/kernels.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, GEMV_SOURCES):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload, batch, prefetch):
    """HBM bytes per algorithmic byte of the kernel class's launches, from the committed
    FETCH_SIZE / WRITE_SIZE counter runs, if those were taken on the kernel source as it is now
    and in the same prefetch mode (else None).  The counter runs event-time every launch, which
    shifts the mix of launch sizes, so the ratio (not their bytes per launch) carries over."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}_b{batch}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "-")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if (kv.get("source_sha256") != source_hash(kernel) or "traffic_bytes_per_launch" not in kv
            or "algo_bytes_per_launch" not in kv or kv.get("prefetch") != ("on" if prefetch else "off")):
        return None
    return float(kv["traffic_bytes_per_launch"]) / float(kv["algo_bytes_per_launch"])


def run_copy_calibration(args):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy-calibration", "copies": args.steps, "bytes_read_per_copy": n,
                      "bytes_written_per_copy": n}), flush=True)


def cache_flags(w, prefetch):
    import expert_offload_lru_amd as moe
    flags = (moe.POOL_SHARED if w["pool_shared"] else 0) | (moe.SHARED_EXPERT if w["shared_expert"] else 0)
    flags |= moe.WAVES_UNION if w.get("waves") == "union" else 0
    flags |= moe.POLICY_LFU if w.get("policy") == "lfu" else 0
    flags |= moe.ADAPTIVE_CAPACITY if w.get("adaptive") else 0
    flags |= moe.PREFETCH if prefetch else 0
    return flags


def build_model(w, seed, prefetch):
    import torch

    import expert_offload_lru_amd as moe
    import synth

    cache = moe.Cache(w["E"], w["K"], w["k"], w["H"], w["I"], w["quant"], w["L"], cache_flags(w, prefetch))
    S = cache.S
    L, E = w["L"], w["E"]
    M = w["distinct"] or L * E
    t = time.time()
    store = moe.HostBuffer(M * S)
    blocks = store.numpy(shape=(M, S))
    keys = [(0, m) for m in range(M)] if w["distinct"] else [(l, e) for l in range(L) for e in range(E)]
    synth.fill_blocks(blocks, seed, w["quant"], w["H"], w["I"], keys)
    block_of = np.empty((L, E), dtype=np.int64)
    for l in range(L):
        for e in range(E):
            block_of[l, e] = synth.alias_index(l, e, E, M) if w["distinct"] else l * E + e
        cache.set_expert_ptrs(l, [store.ptr + int(block_of[l, e]) * S for e in range(E)])
    router_np = synth.router_weights(seed + 1, L, E, w["H"])
    router = torch.from_numpy(router_np).cuda()
    shared = None
    shared_np = None
    if w["shared_expert"]:
        shared_np = synth.shared_expert_blocks(seed, L, w["quant"], w["H"], w["I"])
        shared = torch.from_numpy(shared_np).cuda()
    log(f"generated {M} distinct expert blocks ({M * S / 1e9:.2f} GB pinned) in {time.time() - t:.1f}s")
    return dict(cache=cache, store=store, blocks=blocks, block_of=block_of, router=router, router_np=router_np,
                shared=shared, shared_np=shared_np, S=S)


def require_finite(out, what):
    """A synthetic stack whose residual stream overflowed routes on non-finite inputs, and its
    timing then says nothing about the method: refuse to report it."""
    import torch
    if not bool(torch.isfinite(out).all()):
        raise SystemExit(f"bench: non-finite outputs after the timed {what} steps; the synthetic stack diverged")


def run_steps(w, m, xs, first, n, prefetch):
    """Decode steps through the whole stack; the layer loop runs in the library."""
    import torch
    cache = m["cache"]
    L = w["L"]
    b = xs.shape[1]
    if "router_ptrs" not in m:
        m["router_ptrs"] = [m["router"][l].data_ptr() for l in range(L)]
        m["shared_ptrs"] = [m["shared"][l].data_ptr() for l in range(L)] if m["shared"] is not None else None
    key = "out%d" % b
    if key not in m:
        m[key] = torch.empty(b, w["H"], dtype=torch.float32, device="cuda")
    for step in range(first, first + n):
        cache.stack_forward(xs[step], b, m["router_ptrs"], m[key], shared_ptrs=m["shared_ptrs"])


def new_cache(w, m, prefetch):
    """Another cache over the same host store (a cold start for another batch size)."""
    import expert_offload_lru_amd as moe
    cache = moe.Cache(w["E"], w["K"], w["k"], w["H"], w["I"], w["quant"], w["L"], cache_flags(w, prefetch))
    S = m["S"]
    for l in range(w["L"]):
        cache.set_expert_ptrs(l, [m["store"].ptr + int(m["block_of"][l, e]) * S for e in range(w["E"])])
    if m.get("file_store"):
        cache.set_file_store(*m["file_store"])
    return cache


def prepare_file_store(args, w, m):
    """The two-tier store: the expert blocks in a file, block (layer, e) at (layer * E + e) * S,
    written once from the synthetic host store and dropped from the page cache, so that the
    first read of each block comes from the device."""
    path = args.file_store
    S, L, E = m["S"], w["L"], w["E"]
    if not os.path.exists(path) or os.path.getsize(path) < L * E * S:
        t = time.time()
        with open(path, "wb") as f:
            for l in range(L):
                for e in range(E):
                    f.write(memoryview(m["blocks"][int(m["block_of"][l, e])]))
                if l % 8 == 7:
                    log(f"  expert file: {l + 1} of {L} layers written")
            f.flush()
            os.fsync(f.fileno())
        log(f"wrote the expert file {path}: {L * E * S / 1e9:.2f} GB in {time.time() - t:.1f}s")
    fd = os.open(path, os.O_RDONLY)
    try:
        os.posix_fadvise(fd, 0, 0, os.POSIX_FADV_DONTNEED)
    finally:
        os.close(fd)
    m["file_store"] = (path, args.ram_blocks, args.readers)
    m["cache"].set_file_store(path, args.ram_blocks, args.readers)


# ----------------------------------------------------------------------------- timed windows

_MARK = {}
TIMED_WINDOWS = []          # labels of the marked windows, in order


def mark():
    """A one-element bitwise_not on the current stream: a kernel of its own name that brackets
    a timed window in a kernel trace (two per window, launched outside the timed region)."""
    import torch
    t = _MARK.get("t")
    if t is None:
        t = _MARK["t"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    t.bitwise_not_()


def prime_steps(b):
    """Steps from an empty cache before the steady state: 64 one-token steps (the steady state
    of a 256-step trace is taken to start there), fewer for large batches, whose every step
    touches most experts."""
    return max(16, min(64, 256 // b))


def pick_hit_rate(st):
    buckets = [st["small"], st["large"]]
    picks = sum(bk["picks"] for bk in buckets)
    return round(sum(bk["pick_hits"] for bk in buckets) / picks, 4) if picks else None


def kernel_table(tm):
    """Per kernel class: launches timed, average event duration, GB/s and fraction of HBM peak,
    share of the timed kernel time (every class is sampled with the same stride, so the sampled
    sums compare); and the class with the most time."""
    live = [n for n in KERNEL_NAME if tm[n]["launches"]]
    total = sum(tm[n]["ms"] for n in live)
    kernels = {}
    for name in live:
        kt = tm[name]
        gbs = kt["bytes"] / (kt["ms"] * 1e-3) / 1e9
        kernels[name] = dict(launches=kt["launches"], avg_us=round(kt["ms"] * 1e3 / kt["launches"], 3),
                             algo_bytes_per_launch=round(kt["bytes"] / kt["launches"]), gbs=round(gbs, 1),
                             hbm_frac=round(gbs / HBM_PEAK_GBS, 4), share=round(kt["ms"] / total, 4))
    dom = max(live, key=lambda n: tm[n]["ms"]) if live else None
    return kernels, dom


def measure_decode(args, w, m, cache, batch, warmup, steps, prefetch, mask, label, prime=None, reps=3):
    """The decode protocol for one batch size on one cache: a cold-start window of `prime`
    steps from the empty cache, `warmup` untimed steps, then `reps` timed windows of `steps`
    steps (value: the median window).  Counters and kernel timing cover the timed windows."""
    import torch

    import synth
    prime = prime_steps(batch) if prime is None else prime
    total = prime + warmup + reps * steps
    xs_np = synth.ar1_streams(args.seed + 2, batch, total, w["H"])
    xs = torch.from_numpy(xs_np).cuda()
    torch.cuda.synchronize()
    m["cache"] = cache
    cache.set_prefetch(args.pf_backlog, args.pf_ahead or w["pf_ahead"])
    cache.set_decode_fusion(args.fusion)
    cold = None
    if prime:
        cache.reset_stats()
        t0 = time.perf_counter()
        run_steps(w, m, xs, 0, prime, prefetch)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        st = cache.stats()
        cold = dict(steps=prime, value=round(batch * prime / dt, 2), ms_per_step=round(dt * 1e3 / prime, 4),
                    hit_rate=pick_hit_rate(st), pcie_h2d_gbs_avg=round(st["bytes_h2d_copied"] / dt / 1e9, 2))
    run_steps(w, m, xs, prime, warmup, prefetch)
    torch.cuda.synchronize()
    cache.reset_stats()
    cache.reset_timing()
    cache.set_timing(mask, stride=args.timing_stride)
    times = []
    first = prime + warmup
    for r in range(reps):
        mark()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(w, m, xs, first + r * steps, steps, prefetch)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        mark()
        TIMED_WINDOWS.append(f"{label}-w{r}")
    torch.cuda.synchronize()
    cache.set_timing(0)
    require_finite(m["out%d" % batch], f"decode batch {batch}")
    st = cache.stats()
    tm = cache.timing()
    dt_all = sum(times)
    med = sorted(times)[len(times) // 2]
    tokens = batch * steps
    buckets = [st["small"], st["large"]]
    uh = sum(bk["hits"] for bk in buckets)
    um = sum(bk["misses"] for bk in buckets)
    kernels, dom = kernel_table(tm)
    roof = None
    if dom:
        kt = tm[dom]
        achieved = kt["bytes"] / (kt["ms"] * 1e-3) / 1e9
        algo = kt["bytes"] / kt["launches"]
        ratio = measured_traffic(dom, args.workload, batch, prefetch)
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=round(ratio * algo) if ratio else None,
                    traffic_over_algo=round(ratio, 4) if ratio else None,
                    kernel=KERNEL_NAME[dom], kernel_class=dom, launches=kt["launches"],
                    avg_launch_us=round(kt["ms"] * 1e3 / kt["launches"], 3), algo_bytes_per_launch=round(algo),
                    timing=f"HIP events recorded by the dispatch (hipExtLaunchKernel) on the launch stream, one "
                           f"launch in {args.timing_stride} of each kernel class, over the timed windows")
    # the layer's expert work as a whole: every expert kernel's bytes over their summed time
    ex = [tm[n] for n in ("gate_up_early", "gate_up", "down", "down_early", "expert_fused") if tm[n]["launches"]]
    expert_frac = None
    if ex:
        expert_frac = round(sum(k["bytes"] for k in ex) / (sum(k["ms"] for k in ex) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    capacity = None
    if w.get("adaptive"):
        caps = [cache.layer_capacity(l)[1] for l in range(w["L"])]
        capacity = dict(min=min(caps), max=max(caps), moved=sum(abs(c - w["K"]) for c in caps) // 2)
    return dict(xs_np=xs_np, value=round(tokens / med, 2), ms_per_step=round(med * 1e3 / steps, 4), steps=steps,
                windows_tokens_per_s=[round(tokens / t, 2) for t in times], cold_start=cold,
                adaptive_targets=capacity, warmup=warmup, prime=prime, roofline=roof, kernels=kernels,
                expert_kernels_hbm_frac=expert_frac, hit_rate=pick_hit_rate(st),
                unique_hit_rate=round(uh / (uh + um), 4) if (uh + um) else None,
                pcie_h2d_gbs_avg=round(st["bytes_h2d_copied"] / dt_all / 1e9, 2),
                h2d_bytes_per_token=round(st["bytes_h2d_copied"] / (tokens * reps)),
                waves_per_step=round(st["waves"] / (steps * reps), 3),
                prefetch=dict(issued=st["prefetch_issued"], used=st["prefetch_used"], wasted=st["prefetch_wasted"],
                              candidates=st["prefetch_candidates"], deferred=st["prefetch_deferred"]),
                host_us_per_step={k: round(st["host_" + k + "_us"] / (steps * reps), 1)
                                  for k in ("call", "wait", "plan", "upload", "launch", "prefetch", "event")},
                ram_tier=dict(hits=st["ram_hits"], misses=st["ram_misses"], evictions=st["ram_evictions"],
                              hit_rate=round(st["ram_hits"] / max(1, st["ram_hits"] + st["ram_misses"]), 4),
                              file_read_gbs=round(st["bytes_read_file"] / dt_all / 1e9, 3))
                if st["ram_hits"] + st["ram_misses"] else None)


def warm_all_resident(w, m, prefetch, seed):
    """A K = E cache over the same host store, filled by 32-token steps until every expert of
    every layer holds a slot."""
    import torch

    import synth
    wk = dict(w, K=w["E"])
    cache = new_cache(wk, m, prefetch)
    m["cache"] = cache
    xw = torch.from_numpy(synth.ar1_streams(seed + 9, 32, 64, w["H"])).cuda()
    for warm in range(1, xw.shape[0] + 1):
        run_steps(wk, m, xw, warm - 1, 1, prefetch)
        torch.cuda.synchronize()
        if all(cache.slot_of(l, e) >= 0 for l in range(w["L"]) for e in range(w["E"])):
            return wk, cache, warm
    cache.close()
    raise SystemExit("bench: 64 warm-up steps of 32 tokens did not make every expert resident")


def measure_upper_bound(args, w, m, prefetch, mask, b0):
    """The headline batch with every expert resident (K = E, warmed until every expert holds a
    slot, so nothing is paged in): the regular path, then (one token) captured steps."""
    wk, cache, warm = warm_all_resident(w, m, prefetch, args.seed)
    try:
        reg = measure_decode(args, wk, m, cache, b0, args.warmup, args.steps, prefetch, mask, f"bound-b{b0}",
                             prime=0)
        out = {"slots": w["E"], "warm_32_token_steps": warm,
               "regular": {k: reg[k] for k in ("value", "ms_per_step", "windows_tokens_per_s", "hit_rate",
                                              "pcie_h2d_gbs_avg", "kernels", "expert_kernels_hbm_frac",
                                              "host_us_per_step")}}
        if b0 == 1:
            cache.set_graph(True)
            g = measure_decode(args, wk, m, cache, 1, args.warmup, args.steps, prefetch, 0, "bound-graph-b1",
                               prime=0)
            out["graph"] = {k: g[k] for k in ("value", "ms_per_step", "windows_tokens_per_s", "hit_rate")}
            out["graph"]["graph_steps"] = cache.stats()["graph_steps"]
            out["graph"]["host_us_per_step"] = {k: g["host_us_per_step"][k] for k in ("call", "wait", "plan",
                                                                                      "launch")}
        return out
    finally:
        cache.close()


def link_sweep():
    """Pinned host-to-device copy rate on one stream, for one expert block (2.65 MB) and for
    64 MB copies (SGLang page, "A preflight script before you turn it on": measure the link
    with a pinned-memory copy test)."""
    import torch
    rates = {}
    stream = torch.cuda.Stream()
    for size, n in ((2654208, 48), (64 << 20, 6)):
        src = torch.empty(size, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty(size, dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(stream):
            dst.copy_(src, non_blocking=True)          # first touch of both buffers
            stream.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                dst.copy_(src, non_blocking=True)
            e1.record(stream)
        e1.synchronize()
        rates["%.2f MB" % (size / 1e6)] = round(size * n / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2)
        del src, dst
    return dict(unit="GB/s", copies="pinned host to device, one stream, back to back", rates=rates)


# ----------------------------------------------------------------------------- prefill

def run_prefill(args, w):
    """Prompts of --prompt tokens through every layer (per-layer calls of the prefill path)."""
    import torch

    import expert_offload_lru_amd as moe
    import synth
    if args.prefill_warm:
        w = dict(w, K=w["E"])            # room for every expert of a layer
    m = build_model(w, args.seed, prefetch=False)
    cache = m["cache"]
    L, H = w["L"], w["H"]
    resident = None
    if args.prefill_warm:
        # decode steps of 32 AR(1) streams until every expert of every layer is resident
        xw = torch.from_numpy(synth.ar1_streams(args.seed + 9, 32, 64, H)).cuda()
        for s in range(64):
            run_steps(w, m, xw, s, 1, False)
            torch.cuda.synchronize()
            resident = sum(cache.slot_of(l, e) >= 0 for l in range(L) for e in range(w["E"]))
            if resident == L * w["E"]:
                break
        log(f"prefill: {resident} of {L * w['E']} experts resident after warming")
    xs = [torch.from_numpy(synth.prefill_prompt(args.seed + 5 + i, args.prompt, H)).cuda()
          for i in range(args.warmup + args.steps)]
    bufs = [torch.empty_like(xs[0]), torch.empty_like(xs[0])]

    def prompt(x):
        cur = x
        for l in range(L):
            out = bufs[l & 1]
            cache.forward(l, cur, args.prompt, m["router"][l], out,
                          shared_w=m["shared"][l] if m["shared"] is not None else None, residual=True)
            cur = out

    for i in range(args.warmup):
        prompt(xs[i])
    torch.cuda.synchronize()
    cache.reset_stats()
    cache.reset_timing()
    # gate/up and down launches alternate: an odd stride samples both
    cache.set_timing(moe.TIME_PREFILL, stride=args.timing_stride | 1)
    mark()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        prompt(xs[args.warmup + i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    mark()
    TIMED_WINDOWS.append("prefill")
    cache.set_timing(0)
    require_finite(bufs[(L - 1) & 1], "prefill")
    st = cache.stats()
    tm = cache.timing()["prefill_gemm"]
    tokens = args.prompt * args.steps
    roof = None
    if tm["launches"]:
        achieved = tm["flops"] / (tm["ms"] * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / MFMA_PEAK_TFLOPS, 4), traffic=None,
                    kernel="k_prefill_gemm (grouped fp16 MFMA GEMM, gate/up and down)", launches=tm["launches"],
                    avg_launch_us=round(tm["ms"] * 1e3 / tm["launches"], 3),
                    flops_per_launch=round(tm["flops"] / tm["launches"]))
    pf = st["prefill"]
    result = {
        "metric": "MoE-stack prefill tokens/s", "value": round(tokens / dt, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3 / args.steps, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE[w["quant"]] + "-mfma",
        "data": "synthetic",
        "config": {"workload": args.workload + "-prefill" + ("-warm" if args.prefill_warm else ""), "layers": L,
                   "experts": w["E"], "top_k": w["k"], "hidden": H, "inter": w["I"],
                   "quant": QUANT_NAME[w["quant"]], "slots": w["K"], "prompt_tokens": args.prompt,
                   "experts_resident": resident},
        "roofline": roof,
        "experts_from_slots": pf["hits"], "experts_uploaded": pf["misses"],
        "pcie_h2d_gbs_avg": round(st["bytes_h2d_copied"] / dt / 1e9, 2),
        "h2d_bytes_per_prompt": round(st["bytes_h2d_copied"] / args.steps),
        "host_us_per_layer": {k: round(st["host_" + k + "_us"] / (args.steps * L), 1)
                              for k in ("call", "wait", "plan", "upload", "launch", "event")},
        "timed_windows": TIMED_WINDOWS,
    }
    cache.close()
    m["store"].free()
    print(json.dumps(result), flush=True)


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(w, m, xs_np, budget_s=20.0):
    """The oracle as it stands on whole decode steps of the same stack, its BLAS on every core
    this process may run on."""
    from threadpoolctl import threadpool_limits

    from oracle import ffn, formats, lru, route
    L, E, k = w["L"], w["E"], w["k"]
    cores = len(os.sched_getaffinity(0))
    sim = lru.CacheSim(E, w["K"], k, L, shared_pool=w["pool_shared"], block_bytes=m["S"])
    t0 = time.time()
    tokens = 0
    steps = 0
    with threadpool_limits(limits=cores):
        while steps < xs_np.shape[0]:
            x = xs_np[steps].astype(np.float64)
            for l in range(L):
                ids, gate, _z, _p = route.route(x, m["router_np"][l], k)
                sim.decode(l, ids, steps)
                experts = lambda layer, e: formats.decode_expert(w["quant"], m["blocks"][m["block_of"][layer, e]],
                                                                 w["H"], w["I"])
                shared = None
                if m["shared_np"] is not None:
                    shared = formats.decode_expert(w["quant"], m["shared_np"][l], w["H"], w["I"])
                y = ffn.moe_layer_given_routing(x, ids, gate, experts, layer=l, shared=shared)
                x = x + y
            steps += 1
            tokens += x.shape[0]
            if time.time() - t0 > budget_s:
                break
    dt = time.time() - t0
    return dict(value=tokens / dt, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{steps} decode step(s) x {L} layers, batch {xs_np.shape[1]}, from a cold cache "
                       f"(routing, LRU replay, float64 dequant + SwiGLU), {dt:.1f}s with BLAS on {cores} cores")


# ----------------------------------------------------------------------------- kernel-trace summary

def trace_summary(args):
    """Cut a rocprofv3 kernel trace (CSV) of a bench run down to its timed windows (the kernels
    between each pair of marker kernels) and print, per window group, each kernel's launches,
    average duration and share of the window's kernel time, as a markdown table."""
    with open(args.bench_json) as fh:
        line = [l for l in fh.read().splitlines() if l.startswith("{")][-1]
    labels = json.loads(line)["timed_windows"]
    rows = []
    with open(args.trace) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"], 0.0))
    rows.sort()
    print(f"Timed windows of `{os.path.basename(args.bench_json)}` cut from `{os.path.basename(args.trace)}`"
          f" ({len(labels)} windows between marker kernels).\n")
    for lab, grp in _windows(rows, labels).items():
        g = {}
        for s0, s1, name, _v in grp:
            d = g.setdefault(_short(name), [0, 0])
            d[0] += 1
            d[1] += s1 - s0
        total = sum(v[1] for v in g.values())
        print(f"### {lab}\n\n| kernel | launches | average us | total us | share |\n|---|---|---|---|---|")
        for name, (n, ns) in sorted(g.items(), key=lambda kv: -kv[1][1]):
            print(f"| `{name}` | {n} | {ns / n / 1e3:.3f} | {ns / 1e3:.1f} | {ns / total:.3f} |")
        print()


KERNEL_CLASS_OF = (("k_router", "router"), ("k_expert_gemv_pre", "gate_up_early"),
                   ("k_expert_gemv_stream", "gate_up"), ("k_down_combine_picks", "down_early"),
                   ("k_down_combine", "down"), ("k_expert_fused", "expert_fused"),
                   ("k_combine", "combine"), ("k_prefill_gemm", "prefill_gemm"))


def kernel_class(short):
    """(timing class, whether the kernel starts a timed launch of it) of a library kernel, from its
    name: the router's selection launch belongs to the logits launch before it, the plain GEMV
    goes by its matrix count."""
    if short.startswith("k_router_select"):
        return "router", False
    for prefix, cls in KERNEL_CLASS_OF:
        if short.startswith(prefix):
            return cls, True
    if short.startswith("k_expert_gemv<"):
        return ("gate_up" if short.split(",")[3].strip() == "2" else "down"), True
    return None, False


def _windows(rows, labels):
    """rows: sorted (start, end, name, value); the rows between each pair of marker kernels,
    grouped by window label without its repeat suffix."""
    marks = [i for i, r in enumerate(rows) if "bitwise_not" in r[2]]
    if len(marks) != 2 * len(labels):
        raise SystemExit(f"{len(marks)} marker kernels for {len(labels)} windows")
    groups = {}
    for wi, lab in enumerate(labels):
        a, b = marks[2 * wi], marks[2 * wi + 1]
        groups.setdefault(lab.rsplit("-w", 1)[0], []).extend(rows[a + 1:b])
    return groups


def _short(name):
    return name.replace("moe::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def _counter_rows(path):
    rows, cname = [], None
    with open(path) as fh:
        for r in csv.DictReader(fh):
            cname = r["Counter_Name"]
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows, cname


def counter_summary(args):
    """HBM traffic per launch of each kernel class over the timed windows of two bench runs
    under rocprofv3 --pmc (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled to
    bytes by what the same counter read for the 256 MiB device copy of --mode
    copy-calibration, beside the algorithmic bytes per launch that the FETCH run's event
    timing reports (run it with --timing-stride 1 so every launch is counted); with
    --write-traffic, the ratios go to profiles/traffic_<class>_<workload>_b<batch>.txt, which
    later bench runs scale their own bytes by while the kernel sources are unchanged."""
    paths = args.counters.split(",")
    cals = args.calibration.split(",")
    jsons = args.bench_json.split(",")
    per_counter = []
    for path, cal_path, jpath in zip(paths, cals, jsons):
        with open(jpath) as fh:
            res = json.loads([l for l in fh.read().splitlines() if l.startswith("{")][-1])
        rows, cname = _counter_rows(path)
        cal, _ = _counter_rows(cal_path)
        scale = (256 << 20) / (max(v for *_x, v in cal) * 1024.0)
        by = {}
        for lab, grp in _windows(rows, res["timed_windows"]).items():
            per = by.setdefault(lab, {})
            for _s0, _s1, name, v in grp:
                cls, starts = kernel_class(_short(name))
                if cls:
                    d = per.setdefault(cls, [0, 0.0])
                    d[0] += 1 if starts else 0
                    d[1] += v * 1024.0 * scale
        per_counter.append((cname, scale, by, res))
    (c0, s0, by0, res0) = per_counter[0]
    w = res0["config"]["workload"]
    print(f"HBM traffic per launch over the timed windows (`{w}`): "
          + "; ".join(f"{c} scaled by {s:.4f} bytes per counted KiB (from a 256 MiB device copy)"
                      for c, s, _b, _r in per_counter) + ".\n")
    for lab in by0:
        batch = lab[1:]
        algo = res0.get("by_batch", {}).get(batch, {}).get("kernels", {})
        names = [c for c, *_ in per_counter]
        print(f"### {lab}\n\n| kernel class | launches | " + " | ".join(f"{n} bytes/launch" for n in names)
              + " | algorithmic bytes/launch | traffic / algorithmic |\n|---|---|" + "---|" * len(names) + "---|---|")
        for cls, (n, _t) in sorted(by0[lab].items(), key=lambda kv: -kv[1][1]):
            vals = [b.get(lab, {}).get(cls, [1, 0.0]) for _c, _s, b, _r in per_counter]
            per_launch = [v[1] / v[0] for v in vals]
            total = sum(per_launch)
            al = algo.get(cls, {}).get("algo_bytes_per_launch")
            ratio = total / al if al else None
            print(f"| {cls} | {n} | " + " | ".join(f"{x:.0f}" for x in per_launch)
                  + f" | {al if al else '-'} | {ratio:.3f} |" if ratio else
                  f"| {cls} | {n} | " + " | ".join(f"{x:.0f}" for x in per_launch) + " | - | - |")
            if args.write_traffic and ratio:
                path = os.path.join(ROOT, "profiles", f"traffic_{cls}_{w}_b{batch}.txt")
                with open(path, "w") as fh:
                    fh.write(f"# HBM traffic of the {cls} kernel class, {w}, batch {batch}, timed windows\n")
                    fh.write(f"# commands: {args.commands}\n" if args.commands else "")
                    fh.write(f"kernel_class: {cls}\nworkload: {w}\nbatch: {batch}\n")
                    fh.write(f"prefetch: {'on' if res0['config']['prefetch'] else 'off'}\n")
                    fh.write(f"launches: {n}\n")
                    for (cname, scale, _b, _r), x in zip(per_counter, per_launch):
                        fh.write(f"{cname.lower()}_bytes_per_launch: {x:.0f}\n{cname.lower()}_scale: {scale:.4f}\n")
                    fh.write(f"traffic_bytes_per_launch: {total:.0f}\nalgo_bytes_per_launch: {al}\n")
                    fh.write(f"traffic_over_algo: {ratio:.4f}\nsource_sha256: {source_hash(cls)}\n")
        print()


SIMDS, CUS, CLOCK_GHZ = 1024, 256, 2.4     # MI355X: 256 CUs x 4 SIMDs, peak engine clock


def pmc_summary(args):
    """Per kernel, over the timed windows of bench runs under rocprofv3 --pmc (one or more
    passes, each with its bench JSON): launches, the profiler's average duration, and the
    counters read as utilisation.  SQ cycle counters count quad-cycles (4 clocks); busy
    fractions divide by the kernel's duration at the 2.4 GHz peak clock (a lower clock under
    load would make them larger):
      valu_busy  = SQ_ACTIVE_INST_VALU * 4 / (1024 SIMDs x cycles)
      mfma_busy  = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles)
      VALU/MFMA  = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA
      lds_wait   = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; lds_conflict = SQ_LDS_BANK_CONFLICT /
                   SQ_ACTIVE_INST_LDS
      waves/SIMD = SQ_WAVE_CYCLES * 4 / cycles / 1024   (resident waves, time average)
      wait       = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES     (share of wave time not able to issue)
      ta_busy    = TA_TA_BUSY_sum / (256 CUs x cycles)
      l2_hit     = TCC_HIT / (TCC_HIT + TCC_MISS)
      dram_stall = TCC_EA0_RDREQ_DRAM_CREDIT_STALL per launch (L2 read requests held back by the
                   memory side)
      utcl1_miss = TCP_UTCL1_TRANSLATION_MISS / TCP_UTCL1_REQUEST (L1 TLB)
      l2_lat     = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ (cycles from L1 to L2 and back)"""
    passes = []
    for path, jpath in zip(args.counters.split(","), args.bench_json.split(",")):
        with open(jpath) as fh:
            res = json.loads([l for l in fh.read().splitlines() if l.startswith("{")][-1])
        disp = {}
        with open(path) as fh:
            for r in csv.DictReader(fh):
                d = disp.setdefault(int(r["Dispatch_Id"]), [int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
                                                             r["Kernel_Name"], {}])
                d[3][r["Counter_Name"]] = float(r["Counter_Value"])
        rows = sorted(tuple(v) for v in disp.values())
        agg = {}
        for lab, grp in _windows(rows, res["timed_windows"]).items():
            for s0, s1, name, cnt in grp:
                k = _short(name)
                if not kernel_class(k)[0]:
                    continue
                a = agg.setdefault(lab, {}).setdefault(k, [0, 0.0, {}])
                a[0] += 1
                a[1] += s1 - s0
                for cn, v in cnt.items():
                    a[2][cn] = a[2].get(cn, 0.0) + v
        passes.append(agg)
    labels = list(passes[0])
    cols = [("waves/launch", lambda c, n, cyc: c["SQ_WAVES"] / n if "SQ_WAVES" in c else None, "{:.0f}"),
            ("VALU instr/wave", lambda c, n, cyc: c["SQ_INSTS_VALU"] / c["SQ_WAVES"]
             if "SQ_INSTS_VALU" in c and c.get("SQ_WAVES") else None, "{:.0f}"),
            ("valu_busy", lambda c, n, cyc: c["SQ_ACTIVE_INST_VALU"] * 4 / n / SIMDS / cyc
             if "SQ_ACTIVE_INST_VALU" in c else None, "{:.2f}"),
            ("waves/SIMD", lambda c, n, cyc: c["SQ_WAVE_CYCLES"] * 4 / n / cyc / SIMDS
             if "SQ_WAVE_CYCLES" in c else None, "{:.1f}"),
            ("wait", lambda c, n, cyc: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]
             if "SQ_WAIT_INST_ANY" in c and c.get("SQ_WAVE_CYCLES") else None, "{:.2f}"),
            ("mfma_busy", lambda c, n, cyc: c["SQ_VALU_MFMA_BUSY_CYCLES"] / n / SIMDS / cyc
             if "SQ_VALU_MFMA_BUSY_CYCLES" in c else None, "{:.2f}"),
            ("VALU/MFMA", lambda c, n, cyc: (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"]
             if c.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in c else None, "{:.1f}"),
            ("LDS instr/wave", lambda c, n, cyc: c["SQ_INSTS_LDS"] / c["SQ_WAVES"]
             if "SQ_INSTS_LDS" in c and c.get("SQ_WAVES") else None, "{:.0f}"),
            ("lds_wait", lambda c, n, cyc: c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES"]
             if "SQ_WAIT_INST_LDS" in c and c.get("SQ_WAVE_CYCLES") else None, "{:.2f}"),
            ("lds_conflict", lambda c, n, cyc: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"]
             if "SQ_LDS_BANK_CONFLICT" in c and c.get("SQ_ACTIVE_INST_LDS") else None, "{:.2f}"),
            ("ta_busy", lambda c, n, cyc: c["TA_TA_BUSY_sum"] / n / CUS / cyc if "TA_TA_BUSY_sum" in c else None,
             "{:.2f}"),
            ("l2_hit", lambda c, n, cyc: c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
             if "TCC_HIT_sum" in c and (c["TCC_HIT_sum"] + c.get("TCC_MISS_sum", 0)) else None, "{:.2f}"),
            ("dram_stall/launch", lambda c, n, cyc: c["TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum"] / n
             if "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum" in c else None, "{:.0f}"),
            ("utcl1_miss", lambda c, n, cyc: c["TCP_UTCL1_TRANSLATION_MISS_sum"] / c["TCP_UTCL1_REQUEST_sum"]
             if c.get("TCP_UTCL1_REQUEST_sum") else None, "{:.4f}"),
            ("l2_lat", lambda c, n, cyc: c["TCP_TCC_READ_REQ_LATENCY_sum"] / c["TCP_TCC_READ_REQ_sum"]
             if c.get("TCP_TCC_READ_REQ_sum") else None, "{:.0f}")]
    for lab in labels:
        kernels = sorted(passes[0][lab], key=lambda k: -passes[0][lab][k][1])
        rows_out = []
        for k in kernels:
            n0, t0, _c = passes[0][lab][k]
            vals = {}
            for agg in passes:
                if k not in agg.get(lab, {}):
                    continue
                n, t, cnt = agg[lab][k]
                cyc = t / n * CLOCK_GHZ                      # ns per launch x GHz
                for name, fn, fmt in cols:
                    if name not in vals:
                        v = fn(cnt, n, cyc)
                        if v is not None:
                            vals[name] = fmt.format(v)
            rows_out.append((k, n0, t0 / n0 / 1e3, vals))
        used = [name for name, _f, _m in cols if any(name in r[3] for r in rows_out)]
        print(f"### {lab}\n\n| kernel | launches | average us | " + " | ".join(used) + " |\n|---|---|---|"
              + "---|" * len(used))
        for k, n, us, vals in rows_out:
            print(f"| `{k}` | {n} | {us:.2f} | " + " | ".join(vals.get(u, "-") for u in used) + " |")
        print()


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=192, help="timed steps per window (three windows)")
    ap.add_argument("--warmup", type=int, default=64, help="untimed steps after the cold-start window")
    ap.add_argument("--workload", default="qwen3-30b-a3b-int4", choices=sorted(WORKLOADS))
    ap.add_argument("--batch", type=int, default=None, help="one decode batch size (overrides --batches)")
    ap.add_argument("--batches", default="1,4,32",
                    help="decode batch sizes, comma separated; the first is the headline run")
    ap.add_argument("--slots", type=int, default=None, help="override the workload's cache slots K")
    ap.add_argument("--distinct", type=int, default=None,
                    help="draw only this many distinct expert blocks for the host store (aliased onto the keys)")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-prefetch", action="store_true")
    ap.add_argument("--adaptive", action="store_true",
                    help="per-layer pools that trade capacity by hit rate (defaults of moe_cache_set_adaptive)")
    ap.add_argument("--fusion", action="store_true",
                    help="one fused gate/up + down + combine launch per wave where it applies (default: two)")
    ap.add_argument("--policy", default="lru", choices=["lru", "lfu"],
                    help="slot policy: least recently or least frequently used")
    ap.add_argument("--waves", default="count", choices=["count", "union"],
                    help="decode waves when tokens*top_k > K: K/top_k tokens each, or as many tokens as "
                         "fit by the union of their experts")
    ap.add_argument("--pf-backlog", type=int, default=4,
                    help="speculative uploads only while fewer expert blocks than this are queued on the link")
    ap.add_argument("--pf-ahead", type=int, default=None,
                    help="layers the stack driver routes ahead for speculation (default: the workload's; the "
                         "speculative routers cost E*H*4 bytes each per layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-upper-bound", action="store_true",
                    help="skip the all-resident (K = E) runs of the first batch size")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--kernel-timing", default="all", choices=["all", "none"])
    ap.add_argument("--timing-stride", type=int, default=16,
                    help="event-time one launch in this many of each class (an event-timed launch costs extra host "
                         "time); prefill uses the next odd number")
    ap.add_argument("--mode", default="decode", choices=["decode", "prefill", "copy-calibration", "link",
                                                         "trace-summary", "counter-summary", "pmc-summary"])
    ap.add_argument("--counters", help="counter-summary: counter_collection.csv files of the FETCH_SIZE and "
                                       "WRITE_SIZE bench runs, comma separated; pmc-summary: the files of "
                                       "any counter passes")
    ap.add_argument("--calibration", help="counter-summary: the same counters' files of --mode copy-calibration")
    ap.add_argument("--write-traffic", action="store_true", help="counter-summary: write profiles/traffic_*.txt")
    ap.add_argument("--commands", default=None, help="counter-summary: the commands to record in the traffic files")
    ap.add_argument("--trace", help="trace-summary: the rocprofv3 kernel_trace.csv")
    ap.add_argument("--bench-json", help="trace-summary: the bench output (its last JSON line) of the traced run")
    ap.add_argument("--prompt", type=int, default=2048, help="prefill prompt tokens")
    ap.add_argument("--file-store", default=None,
                    help="two-tier store: write the experts to this file and read them through a RAM LRU")
    ap.add_argument("--ram-blocks", type=int, default=5120, help="RAM blocks of the two-tier store")
    ap.add_argument("--readers", type=int, default=8, help="reader threads of the two-tier store")
    ap.add_argument("--prefill-warm", action="store_true",
                    help="prefill with every expert resident (K = E, warmed by decode steps): no PCIe uploads")
    args = ap.parse_args()
    if args.mode == "trace-summary":
        trace_summary(args)
        return
    if args.mode == "counter-summary":
        counter_summary(args)
        return
    if args.mode == "pmc-summary":
        pmc_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the offloaded MoE layer is a "
              f"single-GPU path; see the sharding design)", file=sys.stderr)
        sys.exit(2)

    import torch

    import expert_offload_lru_amd as moe
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = dict(WORKLOADS[args.workload])
    w["waves"] = args.waves
    w["policy"] = args.policy
    w["adaptive"] = args.adaptive
    if args.slots:
        w["K"] = args.slots
    if args.distinct:
        w["distinct"] = args.distinct
    if args.mode == "copy-calibration":
        run_copy_calibration(args)
        return
    if args.mode == "link":
        print(json.dumps({"mode": "link", **link_sweep()}), flush=True)
        return
    if args.mode == "prefill":
        run_prefill(args, w)
        return
    prefetch = not args.no_prefetch
    batches = [args.batch] if args.batch else [int(b) for b in args.batches.split(",")]
    link = link_sweep()
    m = build_model(w, args.seed, prefetch)
    if args.file_store:
        prepare_file_store(args, w, m)
    mask = {"all": moe.TIME_ROUTER | moe.TIME_GATE_UP | moe.TIME_DOWN | moe.TIME_FUSED | moe.TIME_GATE_UP_EARLY |
                   moe.TIME_DOWN_EARLY,
            "none": 0}[args.kernel_timing]
    runs = {}
    for i, b in enumerate(batches):
        # the first batch size is the headline run; the others time fewer steps per window
        steps, warmup = (args.steps, args.warmup) if i == 0 else (max(16, min(args.steps, 768 // b)),
                                                                  min(args.warmup, max(4, 128 // b)))
        cache = m["cache"] if i == 0 else new_cache(w, m, prefetch)
        log(f"decode: batch {b}, {prime_steps(b)} cold-start steps, {warmup} warmup, 3 x {steps} timed steps")
        runs[b] = measure_decode(args, w, m, cache, b, warmup, steps, prefetch, mask, f"b{b}")
        cache.close()
    r = runs[batches[0]]
    b0 = batches[0]
    result = {
        "metric": METRIC, "value": r["value"], "unit": "tokens/s", "n_gpus": 1, "steps": r["steps"],
        "warmup": r["warmup"], "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE[w["quant"]], "data": "synthetic",
        "config": {"workload": args.workload, "layers": w["L"], "experts": w["E"], "top_k": w["k"],
                   "hidden": w["H"], "inter": w["I"], "quant": QUANT_NAME[w["quant"]],
                   "slots": w["K"], "pool": "shared" if w["pool_shared"] else "per-layer",
                   "shared_expert": w["shared_expert"], "batch": b0, "prefetch": prefetch, "fused_decode": args.fusion,
                   "waves": args.waves, "policy": args.policy, "adaptive_capacity": args.adaptive,
                   "prefetch_backlog": args.pf_backlog, "prefetch_layers_ahead": args.pf_ahead or w["pf_ahead"],
                   "distinct_host_blocks": w["distinct"] or w["L"] * w["E"],
                   "file_store": dict(ram_blocks=args.ram_blocks, readers=args.readers) if args.file_store else None},
        "protocol": (f"value = median of 3 windows of {r['steps']} timed steps (steady state: after "
                     f"{r['prime']} cold-start steps from an empty cache and {r['warmup']} warmup steps); "
                     f"cold_start = the first {r['prime']} steps from the empty cache"),
        "roofline": r["roofline"],
    }
    for k in ("windows_tokens_per_s", "cold_start", "expert_kernels_hbm_frac", "hit_rate", "unique_hit_rate",
              "pcie_h2d_gbs_avg", "h2d_bytes_per_token", "waves_per_step", "prefetch", "host_us_per_step",
              "kernels", "ram_tier"):
        result[k] = r[k]
    result["pcie_link"] = link
    result["by_batch"] = {str(b): {"value": runs[b]["value"], "ms_per_step": runs[b]["ms_per_step"],
                                   "steps": runs[b]["steps"], "windows_tokens_per_s": runs[b]["windows_tokens_per_s"],
                                   "cold_start": runs[b]["cold_start"], "hit_rate": runs[b]["hit_rate"],
                                   "dominant_kernel": runs[b]["roofline"]["kernel_class"] if runs[b]["roofline"]
                                   else None,
                                   "dominant_hbm_frac": runs[b]["roofline"]["frac"] if runs[b]["roofline"] else None,
                                   "gemv_hbm_frac": {n: runs[b]["kernels"][n]["hbm_frac"]
                                                     for n in ("gate_up_early", "gate_up", "down", "down_early",
                                                               "expert_fused")
                                                     if n in runs[b]["kernels"]},
                                   "expert_kernels_hbm_frac": runs[b]["expert_kernels_hbm_frac"],
                                   "kernels": runs[b]["kernels"],
                                   "pcie_h2d_gbs_avg": runs[b]["pcie_h2d_gbs_avg"],
                                   "waves_per_step": runs[b]["waves_per_step"],
                                   "adaptive_targets": runs[b]["adaptive_targets"]} for b in batches}
    if not args.no_upper_bound and w["K"] < w["E"] and not w["pool_shared"] and not args.file_store:
        log(f"decode bound: batch {b0}, K = E = {w['E']}, every expert resident")
        result["upper_bound_all_resident"] = measure_upper_bound(args, w, m, prefetch, mask, b0)
    result["timed_windows"] = TIMED_WINDOWS
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, m, r["xs_np"], args.cpu_budget)
    m["store"].free()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

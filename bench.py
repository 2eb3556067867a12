"""Benchmark: MoE-stack decode tokens/s through the offloaded MoE layers on one MI355X.

A step is one decode step of the whole stack: for a batch of b tokens, every
one of the L layers runs the router, the LRU plan and miss uploads, the
expert GEMVs and the combine (residual chained, x_{l+1} = x_l + y_l).  The
cache starts cold at the first warmup step; the timed steps follow the
warmup steps on the same token streams (AR(1) hidden states, see synth).

Prints one JSON line (the driver's contract) with, in addition, the roofline
of the dominant kernel (the gate/up expert GEMV, timed with HIP events on its
launch stream) and the CPU oracle timed on a bounded sample of the workload.
"""
import argparse
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

WORKLOADS = {
    # Qwen3-30B-A3B-shaped stack (SGLang page, "What does Paged Experts actually do?")
    "qwen3-30b-a3b-int4": dict(L=48, E=128, k=8, H=2048, I=768, quant=1, K=92, pool_shared=False,
                               shared_expert=False, distinct=768, pf_ahead=5),
    # Qwen3.8-Flash-Next-shaped stack, e2m1 + E4M3, shared pool of 2048 slots, shared expert
    "qwen3.8-flash-next-e2m1": dict(L=48, E=512, k=10, H=3072, I=512, quant=2, K=2048, pool_shared=True,
                                    shared_expert=True, distinct=1031, pf_ahead=1),
    "tiny-fp32": dict(L=1, E=16, k=2, H=256, I=128, quant=0, K=8, pool_shared=False, shared_expert=False,
                      distinct=None, pf_ahead=3),
}
QUANT_NAME = {0: "f32", 1: "int4_g32_f16", 2: "e2m1_g16_e4m3"}
DTYPE = {0: "f32", 1: "int4xf16", 2: "e2m1xf16"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


GEMV_SOURCES = ("expert_offload_lru_amd/csrc/expert_gemv.hip", "expert_offload_lru_amd/csrc/kernels.hpp")


def gemv_source_hash():
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload, batch, prefetch):
    """HBM bytes per algorithmic byte of the kernel's launches, from the committed FETCH_SIZE /
    WRITE_SIZE counter runs, if those were taken on the kernel source as it is now and in the same
    prefetch mode (else None).  The counter runs event-time every launch, which shifts the mix of
    launch sizes, so the ratio (not their bytes per launch) carries over to this run."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}_b{batch}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith((" ", "#", "-")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if (kv.get("source_sha256") != gemv_source_hash() or "traffic_bytes_per_launch" not in kv
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


def build_model(w, seed, batch, prefetch):
    import torch

    import expert_offload_lru_amd as moe
    import synth

    flags = (moe.POOL_SHARED if w["pool_shared"] else 0) | (moe.SHARED_EXPERT if w["shared_expert"] else 0)
    flags |= moe.WAVES_UNION if w.get("waves") == "union" else 0
    flags |= moe.POLICY_LFU if w.get("policy") == "lfu" else 0
    flags |= moe.ADAPTIVE_CAPACITY if w.get("adaptive") else 0
    flags |= moe.PREFETCH if prefetch else 0
    cache = moe.Cache(w["E"], w["K"], w["k"], w["H"], w["I"], w["quant"], w["L"], flags)
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
    flags = (moe.POOL_SHARED if w["pool_shared"] else 0) | (moe.SHARED_EXPERT if w["shared_expert"] else 0)
    flags |= moe.WAVES_UNION if w.get("waves") == "union" else 0
    flags |= moe.POLICY_LFU if w.get("policy") == "lfu" else 0
    flags |= moe.ADAPTIVE_CAPACITY if w.get("adaptive") else 0
    flags |= moe.PREFETCH if prefetch else 0
    cache = moe.Cache(w["E"], w["K"], w["k"], w["H"], w["I"], w["quant"], w["L"], flags)
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


def measure_decode(args, w, m, cache, batch, warmup, steps, prefetch, mask):
    """Warmup then timed decode steps of `batch` AR(1) streams through the stack, from a cold cache."""
    import torch

    import synth
    xs_np = synth.ar1_streams(args.seed + 2, batch, warmup + steps, w["H"])
    xs = torch.from_numpy(xs_np).cuda()
    torch.cuda.synchronize()
    m["cache"] = cache
    cache.set_prefetch(args.pf_backlog, args.pf_ahead or w["pf_ahead"])
    cache.set_decode_fusion(args.fusion)
    run_steps(w, m, xs, 0, warmup, prefetch)
    torch.cuda.synchronize()
    cache.reset_stats()
    cache.reset_timing()
    cache.set_timing(mask, stride=args.timing_stride)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(w, m, xs, warmup, steps, prefetch)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    cache.set_timing(0)
    require_finite(m["out%d" % batch], f"decode batch {batch}")
    st = cache.stats()
    tm = cache.timing()
    tokens = batch * steps
    buckets = [st["small"], st["large"]]
    picks = sum(bk["picks"] for bk in buckets)
    pick_hits = sum(bk["pick_hits"] for bk in buckets)
    uh = sum(bk["hits"] for bk in buckets)
    um = sum(bk["misses"] for bk in buckets)
    # the dominant expert kernel: the fused launch where waves fit one launch list, else the
    # gate/up GEMV (both classes are sampled with the same stride, so their sums compare)
    dom = max(("gate_up_early", "expert_fused", "gate_up"), key=lambda n: tm[n]["ms"])
    gu = tm[dom]
    roof = None
    if gu["launches"]:
        achieved = gu["bytes"] / (gu["ms"] * 1e-3) / 1e9
        ratio = measured_traffic(dom, args.workload, batch, prefetch)
        algo = gu["bytes"] / gu["launches"]
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=round(ratio * algo) if ratio else None,
                    traffic_over_algo=round(ratio, 4) if ratio else None,
                    kernel=KERNEL_NAME[dom], launches=gu["launches"],
                    avg_launch_us=round(gu["ms"] * 1e3 / gu["launches"], 3),
                    algo_bytes_per_launch=round(gu["bytes"] / gu["launches"]))
    kernels = {}
    for name in ("router", "gate_up", "gate_up_early", "down", "expert_fused"):
        kt = tm[name]
        if kt["launches"]:
            kernels[name] = dict(launches=kt["launches"], avg_us=round(kt["ms"] * 1e3 / kt["launches"], 3),
                                 gbs=round(kt["bytes"] / (kt["ms"] * 1e-3) / 1e9, 1))
    capacity = None
    if w.get("adaptive"):
        caps = [cache.layer_capacity(l)[1] for l in range(w["L"])]
        capacity = dict(min=min(caps), max=max(caps), moved=sum(abs(c - w["K"]) for c in caps) // 2)
    return dict(xs_np=xs_np, value=round(tokens / dt, 2), ms_per_step=round(dt * 1e3 / steps, 4), steps=steps,
                adaptive_targets=capacity,
                warmup=warmup, roofline=roof, kernels=kernels,
                hit_rate=round(pick_hits / picks, 4) if picks else None,
                unique_hit_rate=round(uh / (uh + um), 4) if (uh + um) else None,
                pcie_h2d_gbs_avg=round(st["bytes_h2d_copied"] / dt / 1e9, 2),
                h2d_bytes_per_token=round(st["bytes_h2d_copied"] / tokens),
                waves_per_step=round(st["waves"] / steps, 3),
                prefetch=dict(issued=st["prefetch_issued"], used=st["prefetch_used"], wasted=st["prefetch_wasted"],
                              candidates=st["prefetch_candidates"], deferred=st["prefetch_deferred"]),
                host_us_per_step={k: round(st["host_" + k + "_us"] / steps, 1)
                                  for k in ("call", "wait", "plan", "upload", "launch", "prefetch", "event")},
                ram_tier=dict(hits=st["ram_hits"], misses=st["ram_misses"], evictions=st["ram_evictions"],
                              hit_rate=round(st["ram_hits"] / max(1, st["ram_hits"] + st["ram_misses"]), 4),
                              file_read_gbs=round(st["bytes_read_file"] / dt / 1e9, 3))
                if st["ram_hits"] + st["ram_misses"] else None)


def measure_graph(args, w, m, prefetch, warmup, steps):
    """b = 1 decode steps with every expert of every layer resident (K = E, warmed by 32-token
    steps), each step replayed as one captured graph (moe_cache_set_graph)."""
    import torch

    import synth
    wk = dict(w, K=w["E"])
    cache = new_cache(wk, m, prefetch)
    m["cache"] = cache
    try:
        xw = torch.from_numpy(synth.ar1_streams(args.seed + 9, 32, 64, w["H"])).cuda()
        warm = 0
        while warm < xw.shape[0]:
            run_steps(wk, m, xw, warm, 1, prefetch)
            torch.cuda.synchronize()
            warm += 1
            if all(cache.slot_of(l, e) >= 0 for l in range(w["L"]) for e in range(w["E"])):
                break
        cache.set_graph(True)
        xs = torch.from_numpy(synth.ar1_streams(args.seed + 2, 1, warmup + steps, w["H"])).cuda()
        run_steps(wk, m, xs, 0, warmup, prefetch)
        torch.cuda.synchronize()
        cache.reset_stats()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(wk, m, xs, warmup, steps, prefetch)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        require_finite(m["out1"], "captured decode steps")
        st = cache.stats()
        return dict(slots=w["E"], value=round(steps / dt, 2), ms_per_step=round(dt * 1e3 / steps, 4),
                    graph_steps=st["graph_steps"], steps=steps, warm_32_token_steps=warm,
                    host_us_per_step={k: round(st["host_" + k + "_us"] / steps, 1) for k in ("call", "wait", "plan",
                                                                                              "launch")})
    finally:
        cache.close()


KERNEL_NAME = {"gate_up_early": "k_expert_gemv_pre (one-token gate/up + SwiGLU of the resident picks, "
                                "launched before the plan)",
               "expert_fused": "k_expert_fused (gate/up + SwiGLU, down + combine, one launch)",
               "gate_up": "k_expert_gemv gate/up (SwiGLU) GEMV"}
MFMA_PEAK_TFLOPS = 2500.0   # dense fp16/bf16 MFMA, MI355X


def run_prefill(args, w):
    """Prompts of --prompt tokens through every layer (per-layer calls of the prefill path)."""
    import torch

    import expert_offload_lru_amd as moe
    import synth
    if args.prefill_warm:
        w = dict(w, K=w["E"])            # room for every expert of a layer
    m = build_model(w, args.seed, args.prompt, prefetch=False)
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
    t0 = time.perf_counter()
    for i in range(args.steps):
        prompt(xs[args.warmup + i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
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
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE[w["quant"]] + "-mfma", "data": "synthetic",
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
    }
    cache.close()
    m["store"].free()
    print(json.dumps(result), flush=True)


def cpu_baseline(w, m, xs_np, budget_s=20.0):
    """The oracle as it stands, one BLAS thread, on whole decode steps of the same stack."""
    from threadpoolctl import threadpool_limits

    from oracle import ffn, formats, lru, route
    L, E, k = w["L"], w["E"], w["k"]
    sim = lru.CacheSim(E, w["K"], k, L, shared_pool=w["pool_shared"], block_bytes=m["S"])
    t0 = time.time()
    tokens = 0
    steps = 0
    with threadpool_limits(limits=1):
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
    return dict(value=tokens / dt, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{steps} decode step(s) x {L} layers, batch {xs_np.shape[1]}, from a cold cache "
                       f"(routing, LRU replay, float64 dequant + SwiGLU), {dt:.1f}s on one core")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=192)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="qwen3-30b-a3b-int4", choices=sorted(WORKLOADS))
    ap.add_argument("--batch", type=int, default=None, help="one decode batch size (overrides --batches)")
    ap.add_argument("--batches", default="1,4,32",
                    help="decode batch sizes, comma separated; the first is the headline run")
    ap.add_argument("--slots", type=int, default=None, help="override the workload's cache slots K")
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
                    help="skip the all-resident (K = E) run of the first batch size")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--kernel-timing", default="gate_up", choices=["gate_up", "all", "none"])
    ap.add_argument("--timing-stride", type=int, default=16,
                    help="event-time one launch in this many (an event-timed launch costs extra host time); "
                         "prefill uses the next odd number")
    ap.add_argument("--mode", default="decode", choices=["decode", "prefill", "copy-calibration"])
    ap.add_argument("--prompt", type=int, default=2048, help="prefill prompt tokens")
    ap.add_argument("--file-store", default=None,
                    help="two-tier store: write the experts to this file and read them through a RAM LRU")
    ap.add_argument("--ram-blocks", type=int, default=5120, help="RAM blocks of the two-tier store")
    ap.add_argument("--readers", type=int, default=8, help="reader threads of the two-tier store")
    ap.add_argument("--prefill-warm", action="store_true",
                    help="prefill with every expert resident (K = E, warmed by decode steps): no PCIe uploads")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the offloaded MoE layer is a "
              f"single-GPU path; see the sharding design)", file=sys.stderr)
        sys.exit(2)

    import torch

    import expert_offload_lru_amd as moe
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = dict(WORKLOADS[args.workload])
    w["waves"] = args.waves
    w["policy"] = args.policy
    w["adaptive"] = args.adaptive
    if args.slots:
        w["K"] = args.slots
    if args.mode == "copy-calibration":
        run_copy_calibration(args)
        return
    if args.mode == "prefill":
        run_prefill(args, w)
        return
    prefetch = not args.no_prefetch
    batches = [args.batch] if args.batch else [int(b) for b in args.batches.split(",")]
    m = build_model(w, args.seed, batches[0], prefetch)
    if args.file_store:
        prepare_file_store(args, w, m)
    first_cache = m["cache"]
    mask = {"gate_up": moe.TIME_GATE_UP | moe.TIME_FUSED | moe.TIME_GATE_UP_EARLY,
            "all": moe.TIME_ROUTER | moe.TIME_GATE_UP | moe.TIME_DOWN | moe.TIME_FUSED | moe.TIME_GATE_UP_EARLY,
            "none": 0}[args.kernel_timing]
    runs = {}
    for i, b in enumerate(batches):
        # the first batch size is the headline run; the others are shorter, each from a cold cache
        # every batch size starts cold and warms up for --warmup steps (64: the steady state the
        # timed steps measure); the other sizes time fewer steps, so the bench stays within minutes
        steps, warmup = (args.steps, args.warmup) if i == 0 else (max(16, min(args.steps, 768 // b)),
                                                                  max(16, min(args.warmup, 512 // b)))
        cache = m["cache"] if i == 0 else new_cache(w, m, prefetch)
        log(f"decode: batch {b}, {warmup} warmup + {steps} timed steps")
        runs[b] = measure_decode(args, w, m, cache, b, warmup, steps, prefetch, mask)
        if i > 0:
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
                   "waves": args.waves, "policy": args.policy, "adaptive_capacity": args.adaptive, "prefetch_backlog": args.pf_backlog, "prefetch_layers_ahead": args.pf_ahead or w["pf_ahead"],
                   "distinct_host_blocks": w["distinct"] or w["L"] * w["E"],
                   "file_store": dict(ram_blocks=args.ram_blocks, readers=args.readers) if args.file_store else None},
        "roofline": r["roofline"],
    }
    for k in ("hit_rate", "unique_hit_rate", "pcie_h2d_gbs_avg", "h2d_bytes_per_token", "waves_per_step", "prefetch",
              "host_us_per_step", "kernels", "ram_tier"):
        result[k] = r[k]
    result["by_batch"] = {str(b): {"value": runs[b]["value"], "ms_per_step": runs[b]["ms_per_step"],
                                   "steps": runs[b]["steps"], "hit_rate": runs[b]["hit_rate"],
                                   "gemv_hbm_frac": runs[b]["roofline"]["frac"] if runs[b]["roofline"] else None,
                                   "pcie_h2d_gbs_avg": runs[b]["pcie_h2d_gbs_avg"],
                                   "waves_per_step": runs[b]["waves_per_step"],
                                   "adaptive_targets": runs[b]["adaptive_targets"]} for b in batches}
    if not args.no_upper_bound and w["K"] < w["E"] and not w["pool_shared"]:
        # the same b = 1 run with every expert resident (K = E): what the path does without page-in
        wk = dict(w, K=w["E"])
        cache = new_cache(wk, m, prefetch)
        log(f"decode upper bound: batch {b0}, K = E = {w['E']}")
        ub = measure_decode(args, wk, m, cache, b0, args.warmup, args.steps, prefetch, mask)
        cache.close()
        result["upper_bound_all_resident"] = {"slots": w["E"], "value": ub["value"], "ms_per_step": ub["ms_per_step"],
                                              "hit_rate": ub["hit_rate"], "pcie_h2d_gbs_avg": ub["pcie_h2d_gbs_avg"]}
        if b0 == 1:
            log(f"decode upper bound, captured steps: K = E = {w['E']}, every expert resident")
            result["upper_bound_all_resident_graph"] = measure_graph(args, w, m, prefetch, args.warmup, args.steps)
    xs_np = r["xs_np"]
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, m, xs_np, args.cpu_budget)
    first_cache.close()
    m["store"].free()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

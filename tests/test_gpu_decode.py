"""GPU parity of the decode path through the C ABI against the oracle.

Routing ids and the cache trace (slots, hits, fills, evictions) must match
the oracle exactly (near ties in the logits, |gap| <= tau, may swap, see
oracle.route); layer outputs must satisfy max|y - y_ref| <= 2e-3 max|y_ref|.
"""
import sys

import numpy as np
import pytest
import torch

import expert_offload_lru_amd as moe
import synth
from oracle import formats
from gpu_harness import Model, check_routing, compare_records, tol_ok

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class DevView:
    """Wraps a raw device address so torch can copy from it."""

    def __init__(self, ptr, nbytes):
        self.__cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "data": (ptr, False), "version": 3}


# ----------------------------------------------------------------------------- decoders

def test_decoders_match_format_definitions():
    say("decoders: e2m1, e4m3, int4 over all byte values")
    codes = torch.arange(256, dtype=torch.uint8, device="cuda")
    out = torch.empty(512, dtype=torch.float32, device="cuda")
    moe.debug_decode(moe.Q_E2M1_E4M3_G16, 0, codes, 256, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(256, 2)
    b = np.arange(256)
    assert np.array_equal(got[:, 0], formats.E2M1_TABLE[b & 15])
    assert np.array_equal(got[:, 1], formats.E2M1_TABLE[b >> 4])
    moe.debug_decode(moe.Q_E2M1_E4M3_G16, 1, codes, 256, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(256, 2)[:, 0].astype(np.float64)
    ref = formats.E4M3_TABLE
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])
    moe.debug_decode(moe.Q_INT4_G32_F16, 0, codes, 256, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(256, 2)
    assert np.array_equal(got[:, 0], (b & 15) - 8.0)
    assert np.array_equal(got[:, 1], (b >> 4) - 8.0)


# ----------------------------------------------------------------------------- runs

def run_stack(model, x0, residual=True, check_every=1, check_y=lambda s, l: True, prefetch=True):
    """Decode steps through all layers; x0: float32 [steps, b, H].  Checks routing and the
    trace at every call and the output where check_y(step, layer).  Returns (outputs, n_near_ties)."""
    sim = model.oracle_sim()
    outs = []
    near = 0
    worst = 0.0
    for step in range(x0.shape[0]):
        x = torch.from_numpy(x0[step]).cuda()
        for layer in range(model.L):
            n0 = len(model.records)
            out = model.forward(layer, x, residual=residual, prefetch=prefetch)
            torch.cuda.synchronize()
            recs = model.records[n0:]
            x_np = x.cpu().numpy()
            gids = np.concatenate([np.array(r["ids"]) for r in recs])
            ggate = np.concatenate([np.array(r["gate"]) for r in recs])
            ids, gate, dev = check_routing(model, layer, x_np, gids, ggate)
            near += dev
            _slots, orecs = sim.decode(layer, ids, step)
            compare_records(orecs, recs, where=(step, layer))
            gslots = np.concatenate([np.array(r["slots"]) for r in recs]).reshape(ids.shape)
            assert np.array_equal(gslots, _slots), (step, layer)
            o_np = out.cpu().numpy()
            if check_y(step, layer):
                y_gpu = o_np.astype(np.float64) - (x_np.astype(np.float64) if residual else 0.0)
                y_ref = model.oracle_y(layer, x_np, ids, gate)
                ok, err, scale = tol_ok(y_gpu, y_ref)
                worst = max(worst, err / scale)
                assert ok, (step, layer, err, scale)
            outs.append(o_np)
            x = out if residual else x
    say(f"  worst max|err|/max|ref| = {worst:.2e}, near-tie deviations {near}")
    return outs, near, sim


def test_tiny_fp32_single_layer_free_running():
    say("tiny: E=16 k=2 H=256 I=128 fp32 K=8 b=1, 64 steps")
    m = Model(16, 8, 2, 256, 128, moe.Q_F32, 1, seed=21)
    x0 = synth.ar1_streams(22, 1, 64, 256)
    try:
        _outs, _near, sim = run_stack(m, x0, residual=False)
        st = m.cache.stats()
        o = sim.stats.b["small"]
        assert (st["small"]["hits"], st["small"]["misses"], st["small"]["evictions"]) == (o["hits"], o["misses"],
                                                                                         o["evictions"])
        assert st["small"]["misses"] > 8            # the pool churned
    finally:
        m.close()


@pytest.mark.parametrize("b,steps", [(1, 16), (4, 8), (32, 3)])
def test_int4_stack_teacher_forced(b, steps):
    say(f"int4 stack: E=128 k=8 H=2048 I=768 K=92 L=3 b={b} steps={steps}")
    m = Model(128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, n_distinct=131, seed=31)
    x0 = synth.ar1_streams(32, b, steps, 2048)
    try:
        run_stack(m, x0, residual=True, check_y=lambda s, l: s % 4 == 0 or s == steps - 1)
        st = m.cache.stats()
        if b == 32:
            assert st["large"]["plans"] == steps * 3 * 3     # three waves of 11/11/10 tokens
    finally:
        m.close()


def test_int4_stack_union_waves_b32():
    say("int4 stack, union waves: E=128 k=8 H=2048 I=768 K=92 L=3 b=32 steps=3")
    m = Model(128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, flags=moe.WAVES_UNION, n_distinct=131, seed=31)
    x0 = synth.ar1_streams(32, 32, 3, 2048)
    try:
        run_stack(m, x0, residual=True, check_y=lambda s, l: True)
        st = m.cache.stats()
        say(f"  {st['waves']} waves for {3 * 3} calls (the count rule takes {3 * 3 * 3})")
        assert st["waves"] < 3 * 3 * 3
    finally:
        m.close()


@pytest.mark.parametrize("b,steps,K,union", [(1, 12, 24, False), (32, 2, 92, True)])
def test_int4_stack_lfu_policy(b, steps, K, union):
    say(f"int4 stack, LFU policy: E=128 k=8 H=2048 I=768 K={K} L=3 b={b} steps={steps} union={union}")
    flags = moe.POLICY_LFU | (moe.WAVES_UNION if union else 0)
    m = Model(128, K, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, flags=flags, n_distinct=131, seed=41)
    x0 = synth.ar1_streams(42, b, steps, 2048)
    try:
        run_stack(m, x0, residual=True, check_y=lambda s, l: s % 4 == 0 or s == steps - 1)
        st = m.cache.stats()
        assert st["small" if b == 1 else "large"]["evictions"] > 0
    finally:
        m.close()


def test_paging_invariance_bitwise():
    say("paging invariance: K = 128, 92, 32 at b=4, E=128 int4, 2 layers")
    x0 = synth.ar1_streams(41, 4, 6, 2048)
    results = []
    for K in (128, 92, 32):
        m = Model(128, K, 8, 2048, 768, moe.Q_INT4_G32_F16, 2, n_distinct=131, seed=42)
        outs = []
        for step in range(x0.shape[0]):
            x = torch.from_numpy(x0[step]).cuda()
            for layer in range(2):
                x = m.forward(layer, x, residual=True)
                outs.append(x.cpu().numpy())
        results.append(np.stack(outs))
        m.close()
    assert np.array_equal(results[0], results[1]) and np.array_equal(results[0], results[2])


def test_e2m1_shared_pool_with_shared_expert():
    say("e2m1: E=512 k=10 H=3072 I=512, shared pool of 40 slots over 3 layers, shared expert, b=1")
    m = Model(512, 40, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 3, flags=moe.POOL_SHARED, n_distinct=67, seed=51,
              shared_expert=True)
    x0 = synth.ar1_streams(52, 1, 10, 3072)
    try:
        _outs, _near, sim = run_stack(m, x0, residual=True, check_y=lambda s, l: s % 3 == 0)
        assert sim.stats.b["small"]["evictions"] > 0
    finally:
        m.close()


def test_slot_contents_after_churn():
    say("independence check: every resident slot holds its expert's bytes")
    m = Model(32, 6, 2, 256, 256, moe.Q_INT4_G32_F16, 2, seed=61)
    x0 = synth.ar1_streams(62, 3, 12, 256)
    try:
        for step in range(12):
            x = torch.from_numpy(x0[step]).cuda()
            for layer in range(2):
                x = m.forward(layer, x, residual=True)
        torch.cuda.synchronize()
        n_checked = 0
        for layer in range(2):
            for e in range(32):
                s = m.cache.slot_of(layer, e)
                if s < 0:
                    continue
                dev = torch.as_tensor(DevView(m.cache.slot_ptr(layer, s), m.S), device="cuda")
                assert np.array_equal(dev.cpu().numpy(), m.blocks[m.block_of[layer, e]]), (layer, e, s)
                n_checked += 1
        assert n_checked == 2 * 6
    finally:
        m.close()


def test_prefetch_changes_timing_not_results():
    say("prefetch: same outputs and traces with and without speculative uploads")
    x0 = synth.ar1_streams(71, 1, 8, 2048)
    res = []
    for pf in (False, True):
        m = Model(128, 24, 8, 2048, 768, moe.Q_INT4_G32_F16, 4, n_distinct=131, seed=72, prefetch=pf)
        outs = []
        for step in range(x0.shape[0]):
            x = torch.from_numpy(x0[step]).cuda()
            for layer in range(4):
                x = m.forward(layer, x, residual=True, prefetch=pf)
                outs.append(x.cpu().numpy())
        recs = [(r["layer"], r["hits"], r["fills"], r["evictions"]) for r in m.records]
        res.append((np.stack(outs), recs, m.cache.stats()))
        m.close()
    assert np.array_equal(res[0][0], res[1][0])
    assert res[0][1] == res[1][1]
    st = res[1][2]
    assert st["prefetch_issued"] > 0 and st["prefetch_used"] > 0
    assert st["bytes_d2d_copied"] == st["prefetch_used"] * moe.expert_bytes(moe.Q_INT4_G32_F16, 2048, 768)


def test_error_paths_on_gpu():
    say("error paths")
    c = moe.Cache(16, 8, 2, 256, 256, moe.Q_INT4_G32_F16, 2, 0)
    x = torch.zeros(1, 256, device="cuda")
    out = torch.empty_like(x)
    rw = torch.zeros(16, 256, device="cuda")
    assert c.forward_rc(0, x, 1, rw, out) == moe.ERR_NOT_READY
    host = np.zeros(16 * c.S, dtype=np.uint8)                      # pageable: refused
    with pytest.raises(moe.MoeError) as ei:
        c.set_layer(0, host)
    assert ei.value.code == moe.ERR_INVALID
    assert c.forward_rc(0, x, 1, rw, x) == moe.ERR_INVALID        # out aliases x
    assert c.forward_rc(9, x, 1, rw, out) == moe.ERR_INVALID
    c.close()
    c = moe.Cache(16, 8, 2, 256, 256, moe.Q_INT4_G32_F16, 1, moe.SHARED_EXPERT)
    buf = moe.HostBuffer(16 * c.S)
    c.set_layer(0, buf.ptr)
    assert c.forward_rc(0, x, 1, rw, out) == moe.ERR_INVALID       # shared expert weights missing
    c.close()
    buf.free()


def test_zero_input_ties_and_zero_tokens():
    """x = 0: every logit is 0, so the top-k is experts 0 .. k-1 (lowest index first) with gates
    1/E, every expert FFN of 0 is exactly 0 (the int4 offset terms included), and the residual
    output is exactly 0.  A call with no tokens does nothing."""
    say("degenerate: x = 0, E=64 k=4 int4 + shared expert, b=3; zero tokens")
    m = Model(64, 16, 4, 512, 256, moe.Q_INT4_G32_F16, 1, seed=181, shared_expert=True)
    try:
        x = torch.zeros(3, 512, device="cuda")
        out = m.forward(0, x, residual=True)
        torch.cuda.synchronize()
        r = m.records[-1]
        assert np.array_equal(np.array(r["ids"]).reshape(3, 4), np.tile(np.arange(4), (3, 1)))
        assert np.all(np.array(r["gate"], dtype=np.float64) == np.float32(1.0 / 64))
        assert r["fills"] == [(e, e) for e in range(4)] and r["hits"] == []
        assert torch.count_nonzero(out).item() == 0
        n = len(m.records)
        assert m.cache.forward_rc(0, x, 0, m.router[0], torch.empty_like(x), shared_w=m.shared[0]) == moe.OK
        assert len(m.records) == n
    finally:
        m.close()


@pytest.mark.parametrize("K", [16, 1024])
def test_maximum_experts_top_k_and_tokens(K):
    """E = 1024 experts, top_k = 16, 32 tokens: with K = 16 every token is a wave of its own
    (32 plans a call); with K = 1024 one wave of 512 picks, more pairs than one launch list."""
    say(f"maximum sizes: E=1024 k=16 H=256 I=256 int4 b=32 K={K}")
    m = Model(1024, K, 16, 256, 256, moe.Q_INT4_G32_F16, 2, n_distinct=97, seed=190)
    x0 = synth.ar1_streams(191, 32, 2, 256)
    try:
        run_stack(m, x0, residual=True)
        st = m.cache.stats()
        assert st["waves"] == (2 * 2 * 32 if K == 16 else 2 * 2)
    finally:
        m.close()


@pytest.mark.parametrize("union", [False, True])
def test_identical_tokens_wave_rules(union):
    """32 identical tokens route alike: the union rule plans them in one wave, the count rule in
    b*k/K waves of K/k tokens; traces as the oracle's either way."""
    say(f"identical tokens: E=64 k=8 K=32 b=32 union={union}")
    m = Model(64, 32, 8, 512, 256, moe.Q_INT4_G32_F16, 2, seed=195, flags=moe.WAVES_UNION if union else 0)
    row = synth.ar1_streams(196, 1, 3, 512)
    x0 = np.repeat(row, 32, axis=1)
    try:
        run_stack(m, x0, residual=True)
        assert m.cache.stats()["waves"] == 3 * 2 * (1 if union else 8)
    finally:
        m.close()


def test_full_size_qwen3_30b_shape_b1():
    say("full size: L=48 E=128 k=8 H=2048 I=768 int4 K=92/layer b=1, 24 steps, all outputs of steps 0 and 23")
    m = Model(128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 48, n_distinct=131, seed=81)
    x0 = synth.ar1_streams(82, 1, 24, 2048)
    sampled = {(0, 0), (0, 47), (5, 13), (11, 30), (17, 7), (23, 46), (23, 23)}
    try:
        run_stack(m, x0, residual=True, check_y=lambda s, l: s in (0, 23) or (s, l) in sampled)
        st = m.cache.stats()["small"]
        assert st["plans"] == 24 * 48 and st["picks"] == 24 * 48 * 8
    finally:
        m.close()


def test_full_size_qwen3_30b_shape_b32():
    say("full size: L=48 E=128 k=8 H=2048 I=768 int4 K=92/layer b=32, 2 steps, all outputs of step 0")
    m = Model(128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 48, n_distinct=131, seed=91)
    x0 = synth.ar1_streams(92, 32, 2, 2048)
    try:
        run_stack(m, x0, residual=True, check_y=lambda s, l: s == 0 or (s, l) in {(1, 0), (1, 47)})
        assert m.cache.stats()["large"]["plans"] == 2 * 48 * 3
    finally:
        m.close()


def test_full_size_flash_next_shape_b1():
    say("full size: L=48 E=512 k=10 H=3072 I=512 e2m1, shared pool K=2048, shared expert, b=1, 8 steps, "
        "all outputs of steps 0 and 7")
    m = Model(512, 2048, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 48, flags=moe.POOL_SHARED, n_distinct=131, seed=191,
              shared_expert=True)
    x0 = synth.ar1_streams(192, 1, 8, 3072)
    sampled = {(0, 0), (0, 47), (3, 20), (7, 5), (7, 46)}
    try:
        run_stack(m, x0, residual=True, check_y=lambda s, l: s in (0, 7) or (s, l) in sampled)
        st = m.cache.stats()["small"]
        assert st["plans"] == 8 * 48 and st["picks"] == 8 * 48 * 10 and st["hits"] > 0
    finally:
        m.close()


@pytest.mark.parametrize("b,prefetch", [(1, True), (4, False), (24, True)])
def test_int4_stack_adaptive_capacity(b, prefetch):
    """Per-layer pools trading capacity: slots are numbered over all layers, so a layer's
    experts may sit in another layer's original slots; traces bit-exact against the oracle,
    outputs within tolerance, capacities as the oracle's."""
    ad = dict(period=3, delta=2, pairs=2, floor=12)
    L = 4
    say(f"adaptive capacity: E=64 K=24/layer k=4 H=512 I=256 int4 L={L} b={b} prefetch={prefetch}")
    m = Model(64, 24, 4, 512, 256, moe.Q_INT4_G32_F16, L, seed=171 + b, prefetch=prefetch, adaptive=ad)
    x0 = synth.ar1_streams(172 + b, b, 30, 512)
    try:
        _outs, _near, sim = run_stack(m, x0, residual=True, check_y=lambda s, l: s % 3 == 0)
        caps = [m.cache.layer_capacity(l) for l in range(L)]
        assert caps == [(len(sim.adaptive.lists[l]), sim.adaptive.target[l]) for l in range(L)]
        assert sim.adaptive.rebalances >= 8 and [t for _h, t in caps] != [24] * L
        moved = any(s // 24 != l for l in range(L) for s in sim.adaptive.lists[l])
        assert moved                                   # some layer holds another layer's slot
        say(f"  capacities (held, target): {caps}")
    finally:
        m.close()


PRE_CASES = {
    # E, K, k, H, I, quant, L, flags, n_distinct, shared_expert, adaptive
    "int4-per-layer": (128, 40, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, 0, 131, False, None),
    "e2m1-shared-pool": (512, 120, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 3, moe.POOL_SHARED, 131, True, None),
    "f32": (16, 8, 2, 256, 128, moe.Q_F32, 2, 0, None, False, None),
    "int4-adaptive": (64, 16, 4, 512, 256, moe.Q_INT4_G32_F16, 3, 0, None, False,
                      dict(period=2, delta=2, pairs=1, floor=8)),
}


@pytest.mark.parametrize("case", sorted(PRE_CASES))
def test_early_gate_up_bitwise_equals_planned_launches(case):
    """One-token calls launch the resident picks' gate/up and down + combine before the plan.
    Against the same cache without them: outputs and traces bitwise equal, over one-token steps, then steps of 4
    and 24 tokens (whose plans leave the device slot table stale where they change more than
    one launch carries), then one-token steps again."""
    E, K, k, H, I, quant, L, flags, nd, shx, ad = PRE_CASES[case]
    say(f"early gate/up vs planned launches: {case}")
    sched = [1] * 6 + [4] * 2 + [24] + [1] * 6
    runs = []
    for pre in (True, False):
        m = Model(E, K, k, H, I, quant, L, flags=flags, n_distinct=nd, seed=320, shared_expert=shx, prefetch=True,
                  adaptive=ad)
        try:
            m.cache.set_prelaunch(pre)
            m.cache.set_timing(moe.TIME_GATE_UP | moe.TIME_GATE_UP_EARLY | moe.TIME_DOWN_EARLY, stride=1)
            outs = []
            for st, b in enumerate(sched):
                x = torch.from_numpy(synth.ar1_streams(330 + st, b, 1, H)[0]).cuda()
                for layer in range(L):
                    x = m.forward(layer, x, residual=True)
                    outs.append(x.cpu().numpy())
            torch.cuda.synchronize()
            tm = m.cache.timing()
            runs.append((outs, [dict(r) for r in m.records],
                         (tm["gate_up_early"]["launches"], tm["gate_up"]["launches"], tm["down_early"]["launches"])))
        finally:
            m.close()
    (o1, r1, n1), (o0, r0, n0) = runs
    for i, (a, c) in enumerate(zip(o1, o0)):
        assert np.array_equal(a, c), (case, i, float(np.max(np.abs(a - c))))
    compare_records(r1, r0, where=case)
    assert n1[0] == 12 * L and n0[0] == 0          # one early gate/up per one-token call
    assert 0 < n1[2] <= 12 * L and n0[2] == 0      # and, where likely to complete the layer, its down
    say(f"  gate/up launches (early, planned): {n1} with the early launch, {n0} without")


FUSED_SHAPES = {
    # E, K, k, H, I, quant, L, flags, n_distinct, shared_expert, batches
    "f32": (16, 8, 2, 256, 128, moe.Q_F32, 2, 0, None, False, (1, 2)),
    "int4": (128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, 0, 131, False, (1, 2)),
    "e2m1-shared": (512, 400, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 3, moe.POOL_SHARED, 131, True, (1,)),
}


@pytest.mark.parametrize("shape", sorted(FUSED_SHAPES))
def test_fused_decode_launch_bitwise_equals_two_kernels(shape):
    E, K, k, H, I, quant, L, flags, nd, shx, batches = FUSED_SHAPES[shape]
    say(f"fused vs split decode launches: {shape} E={E} K={K} k={k} H={H} I={I} L={L} b={batches}")
    for b in batches:
        steps = 6
        x0 = synth.ar1_streams(301 + b, b, steps, H)
        runs = []
        for fuse in (True, False):
            m = Model(E, K, k, H, I, quant, L, flags=flags, n_distinct=nd, seed=300, shared_expert=shx, prefetch=True)
            try:
                m.cache.set_decode_fusion(fuse)
                m.cache.set_timing(moe.TIME_FUSED | moe.TIME_GATE_UP, stride=1)
                outs = []
                for st in range(steps):
                    x = torch.from_numpy(x0[st]).cuda()
                    for layer in range(L):
                        x = m.forward(layer, x, residual=True)
                        outs.append(x.cpu().numpy())
                torch.cuda.synchronize()
                tm = m.cache.timing()
                runs.append((outs, [dict(r) for r in m.records], tm, m.cache.stats()))
            finally:
                m.close()
        (o_f, r_f, t_f, s_f), (o_s, r_s, t_s, s_s) = runs
        assert t_f["expert_fused"]["launches"] > 0 and t_s["expert_fused"]["launches"] == 0, (b, t_f, t_s)
        assert len(o_f) == len(o_s)
        for i, (a, c) in enumerate(zip(o_f, o_s)):
            assert np.array_equal(a, c), (b, i, float(np.max(np.abs(a - c))))
        compare_records(r_f, r_s, where=(shape, b))
        assert s_f["prefetch_used"] > 0 or s_f["small"]["misses"] > 0
        say(f"  b={b}: {t_f['expert_fused']['launches']} fused launches, {t_f['gate_up']['launches']} split gate/up")


@pytest.mark.parametrize("b", [1, 2])
def test_stack_driver_matches_layer_calls_bitwise(b):
    """moe_stack_forward with and without layer_inputs, and chained moe_layer_forward calls:
    outputs, captured inputs and plan records bitwise equal.  At one token the stack driver
    launches each layer's router and early gate/up ahead; the layer calls do not."""
    say(f"stack driver: moe_stack_forward (with and without layer inputs) == chained moe_layer_forward calls, b={b}")
    x0 = synth.ar1_streams(101, b, 5, 2048)
    L = 4

    def model():
        return Model(128, 40, 8, 2048, 768, moe.Q_INT4_G32_F16, L, n_distinct=131, seed=102, prefetch=True)

    m = model()
    per_layer, ins_ref = [], []
    for step in range(x0.shape[0]):
        x = torch.from_numpy(x0[step]).cuda()
        for layer in range(L):
            ins_ref.append(x.cpu().numpy())
            x = m.forward(layer, x, residual=True, prefetch=True)
        per_layer.append(x.cpu().numpy())
    recs_a = [(r["layer"], r["ids"], r["slots"], r["hits"], r["fills"], r["evictions"]) for r in m.records]
    m.close()
    runs = []
    for with_inputs in (True, False):
        m = model()
        ptrs = [m.router[l].data_ptr() for l in range(L)]
        stacked, ins = [], []
        for step in range(x0.shape[0]):
            x = torch.from_numpy(x0[step]).cuda()
            out = torch.empty_like(x)
            cap = torch.empty(L, b, 2048, device="cuda") if with_inputs else None
            m.cache.stack_forward(x, b, ptrs, out, layer_inputs=cap)
            torch.cuda.synchronize()
            stacked.append(out.cpu().numpy())
            if with_inputs:
                ins.extend(list(cap.cpu().numpy()))
        runs.append((stacked, ins, [(r["layer"], r["ids"], r["slots"], r["hits"], r["fills"], r["evictions"])
                                    for r in m.records]))
        m.close()
    (st_a, ins_a, rec_b), (st_b, _ins_b, rec_c) = runs
    assert np.array_equal(np.stack(per_layer), np.stack(st_a))
    assert np.array_equal(np.stack(per_layer), np.stack(st_b))
    assert np.array_equal(np.stack(ins_ref), np.stack(ins_a))
    assert recs_a == rec_b == rec_c


@pytest.mark.parametrize("quant,E,k,H,I,K_big,K_small,shared", [
    (moe.Q_INT4_G32_F16, 128, 8, 1024, 512, 200, 128, False),
    (moe.Q_E2M1_E4M3_G16, 64, 4, 512, 256, 160, 64, True),
])
def test_waves_beyond_one_launch_list(quant, E, k, H, I, K_big, K_small, shared):
    """b=32 calls whose (first) wave holds more pairs than one launch list: that wave takes the
    unit-tiled down GEMV and a combine of its own tokens, a following small wave the fused
    down+combine.  Outputs match the oracle, and bitwise a cache whose waves all fit one list."""
    say(f"waves beyond one list: quant={quant} E={E} k={k} H={H} I={I} b=32, K={K_big} vs {K_small}")
    x0 = synth.ar1_streams(141, 32, 3, H)
    res = []
    for K in (K_big, K_small):
        m = Model(E, K, k, H, I, quant, 2, flags=moe.POOL_SHARED, seed=142, shared_expert=shared)
        try:
            outs, _near, _sim = run_stack(m, x0, residual=True)
            res.append(np.stack(outs))
        finally:
            m.close()
    assert np.array_equal(res[0], res[1])


@pytest.mark.parametrize("E,b", [(64, 2), (64, 3), (64, 5), (64, 9), (18, 1), (18, 6)])
def test_router_launch_shapes(E, b):
    """Routing and outputs for every router launch shape: one launch for up to four tokens
    (E a multiple of 4), token blocks of 8 and 32 in the two-launch path, and expert counts
    that are not a multiple of 4 (always two launches)."""
    say(f"router shapes: E={E} k=4 H=512 I=256 int4, b={b}")
    m = Model(E, 16, 4, 512, 256, moe.Q_INT4_G32_F16, 2, seed=150 + E + b)
    x0 = synth.ar1_streams(151 + b, b, 4, 512)
    try:
        run_stack(m, x0, residual=True)
    finally:
        m.close()


@pytest.mark.parametrize("b", [1, 4, 9])
def test_router_near_ties_order_exactly(b):
    """Router rows in twins: in three of four pairs one weight of the second row is one ulp
    away, in the fourth the rows are equal.  The top logits then come in pairs about 1e-9 apart
    (relative), closer than the selection's first pass on the upper 32 key bits resolves, so
    it takes the rounds on the whole keys; the order must be the oracle's exactly (the pairs
    are far outside float64 summation error, so no near-tie allowance), equal rows to the
    lower index.  b = 1 and 4: the one-launch router; b = 9: logits and selection launches."""
    say(f"router near ties: E=64 k=4 H=512 I=256 int4, twin rows, b={b}")
    m = Model(64, 16, 4, 512, 256, moe.Q_INT4_G32_F16, 1, seed=160 + b)
    try:
        w = m.router_np[0]
        for i in range(0, 64, 2):
            w[i + 1] = w[i]
            if i % 8 != 0:
                h = (i * 37) % 512
                w[i + 1, h] = np.nextafter(w[i, h], np.float32(np.inf if i % 4 else -np.inf))
        m.router[0].copy_(torch.from_numpy(w))
        x0 = synth.ar1_streams(161 + b, b, 4, 512)
        # the premise: near pairs (equal in the upper 32 key bits) and equal pairs reach the top k + 1
        n_near = n_equal = 0
        for step in range(x0.shape[0]):
            _ids, _gate, z, _p = m.oracle_route(0, x0[step])
            for zt in z:
                top = np.sort(zt)[::-1][:5]
                d = np.abs(np.diff(top))
                n_near += int(np.sum((d > 0) & (d < 1e-6 * np.abs(top[1:]))))
                n_equal += int(np.sum(d == 0))
        assert n_near > 0 and n_equal > 0, (n_near, n_equal)
        _outs, near, _sim = run_stack(m, x0, residual=False)
        assert near == 0
    finally:
        m.close()


def test_speculation_settings_change_timing_not_results():
    say("stack driver: outputs and traces bitwise equal for every speculation depth and queue limit")
    x0 = synth.ar1_streams(181, 1, 6, 2048)
    L = 7
    runs = []
    for pf, backlog, ahead in ((False, 4, 3), (True, 0, 1), (True, 4, 3), (True, 4, 5), (True, 32, 5), (True, 1, 2)):
        m = Model(128, 24, 8, 2048, 768, moe.Q_INT4_G32_F16, L, n_distinct=131, seed=182, prefetch=pf)
        m.cache.set_prefetch(backlog, ahead)
        ptrs = [m.router[l].data_ptr() for l in range(L)]
        outs = []
        for step in range(x0.shape[0]):
            x = torch.from_numpy(x0[step]).cuda()
            out = torch.empty_like(x)
            m.cache.stack_forward(x, 1, ptrs, out)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        recs = [(r["layer"], r["hits"], r["fills"], r["evictions"]) for r in m.records]
        st = m.cache.stats()
        runs.append((np.stack(outs), recs, st["prefetch_issued"]))
        m.close()
        say(f"  prefetch={pf} backlog={backlog} ahead={ahead}: {st['prefetch_issued']} speculative uploads")
    for outs, recs, _ in runs[1:]:
        assert np.array_equal(runs[0][0], outs)
        assert runs[0][1] == recs
    assert runs[1][2] == 0                       # a queue limit of 0 issues nothing
    assert all(r[2] > 0 for r in runs[2:])
    m = Model(16, 8, 2, 256, 128, moe.Q_F32, 1, seed=183)
    try:
        for backlog, ahead in ((4, 6), (4, 0), (-1, 3), (33, 3)):
            with pytest.raises(moe.MoeError):
                m.cache.set_prefetch(backlog, ahead)
    finally:
        m.close()

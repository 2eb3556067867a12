"""Captured decode steps (moe_cache_set_graph) through the C ABI.

Once every expert of every layer holds a slot, a one-token stack step runs as one
replayed HIP graph whose kernels read their units on the device.  Against the same
cache on the regular path: outputs bitwise equal, the same plan records (ids, gates,
slots, hits, fills, evictions), counters and last routing; the records also replay
exactly through the oracle's LRU.
"""
import sys

import numpy as np
import pytest
import torch

import expert_offload_lru_amd as moe
import synth
from gpu_harness import Model

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # E, K, k, H, I, quant, L, flags, n_distinct, shared_expert
    "int4": (128, 128, 8, 2048, 768, moe.Q_INT4_G32_F16, 4, 0, 131, False),
    "e2m1-shared-pool": (128, 384, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 3, moe.POOL_SHARED, 131, True),
    "f32-spare-slots": (16, 20, 2, 256, 128, moe.Q_F32, 2, 0, None, False),
    "int4-not-all-resident": (128, 40, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, 0, 131, False),
    # the 48-layer Qwen3-30B-A3B shape the bench's captured-step figure runs
    "int4-48-layers": (128, 128, 8, 2048, 768, moe.Q_INT4_G32_F16, 48, 0, 131, False),
}

# one-token steps, a 4-token step (regular path) between them; the output buffer index of
# each step (a new buffer makes the cache capture again)
SCHED = [(1, 0), (1, 1), (1, 0), (1, 1), (1, 0), (4, 0), (1, 1), (1, 0), (1, 2), (1, 2), (1, 1)]


def _all_resident(m):
    return all(m.cache.slot_of(l, e) >= 0 for l in range(m.L) for e in range(m.E))


def _run(case, graph):
    E, K, k, H, I, quant, L, flags, nd, shx = CASES[case]
    m = Model(E, K, k, H, I, quant, L, flags=flags, n_distinct=nd, seed=611, shared_expert=shx, prefetch=True)
    try:
        m.cache.set_graph(graph)
        rp = [m.router[l].data_ptr() for l in range(L)]
        sp = [m.shared[l].data_ptr() for l in range(L)] if shx else None
        warm = 0
        if K >= E:
            # 32-token steps of independent streams until every expert of every layer is resident
            xw = synth.ar1_streams(612, 32, 40, H)
            while not _all_resident(m):
                assert warm < xw.shape[0], "warm-up did not make every expert resident"
                x = torch.from_numpy(xw[warm]).cuda()
                m.cache.stack_forward(x, 32, rp, torch.empty_like(x), shared_ptrs=sp)
                torch.cuda.synchronize()
                warm += 1
        n_rec = len(m.records)
        outs = {b: [torch.empty(b, H, device="cuda") for _ in range(3)] for b in (1, 4)}
        res = []
        for s, (b, oi) in enumerate(SCHED):
            x = torch.from_numpy(synth.ar1_streams(620 + s, b, 1, H)[0]).cuda()
            out = outs[b][oi]
            m.cache.stack_forward(x, b, rp, out, shared_ptrs=sp)
            torch.cuda.synchronize()
            res.append(out.cpu().numpy().copy())
        st = m.cache.stats()
        ids, gate = m.cache.last_routing(1)
        return dict(outs=res, recs=[dict(r) for r in m.records], n_warm_recs=n_rec, stats=st,
                    last=(np.array(ids).copy(), np.array(gate).copy()), warm=warm, sim=m.oracle_sim())
    finally:
        m.close()


def _calls(recs):
    """Group plan records into calls (a call's waves follow each other with t0 rising from 0)."""
    calls = []
    for r in recs:
        if r["t0"] == 0:
            calls.append([])
        calls[-1].append(r)
    return calls


@pytest.mark.parametrize("case", sorted(CASES))
def test_captured_steps_bitwise_equal_regular_path(case):
    E, K, k, H, I, quant, L, flags, nd, shx = CASES[case]
    say(f"captured steps vs regular path: {case} E={E} K={K} k={k} H={H} I={I} L={L}")
    g = _run(case, True)
    r = _run(case, False)
    assert g["warm"] == r["warm"]
    for i, (a, c) in enumerate(zip(g["outs"], r["outs"])):
        assert np.array_equal(a, c), (case, i, float(np.max(np.abs(a - c))))
        assert np.all(np.isfinite(a))
    assert len(g["recs"]) == len(r["recs"])
    for i, (a, c) in enumerate(zip(g["recs"], r["recs"])):
        assert a == c, (case, i)
    for key in ("small", "large", "waves", "forwards"):
        assert g["stats"][key] == r["stats"][key], (case, key)
    assert np.array_equal(g["last"][0], r["last"][0]) and np.array_equal(g["last"][1], r["last"][1])
    n_one = sum(1 for b, _ in SCHED if b == 1)
    want = n_one if K >= E else 0
    assert g["stats"]["graph_steps"] == want and r["stats"]["graph_steps"] == 0, (case, g["stats"]["graph_steps"])
    # the records replay exactly through the oracle's LRU (routing ids as the GPU chose them)
    sim = g["sim"]
    for step, call in enumerate(_calls(g["recs"])):
        layer = call[0]["layer"]
        ids = np.concatenate([np.array(rr["ids"]) for rr in call]).reshape(-1, k)
        slots, orecs = sim.decode(layer, ids, step)
        assert len(orecs) == len(call), (case, step)
        for ro, rg in zip(orecs, call):
            assert ro["hits"] == rg["hits"] and ro["fills"] == [tuple(f) for f in rg["fills"]], (case, step)
            assert ro["evictions"] == [tuple(e) for e in rg["evictions"]], (case, step)
        gs = np.concatenate([np.array(rr["slots"]) for rr in call]).reshape(ids.shape)
        assert np.array_equal(gs, slots), (case, step)
    say(f"  {g['warm']} warm-up steps, {g['stats']['graph_steps']} captured steps, records {len(g['recs'])}")


def test_captured_steps_refused_with_adaptive_capacity():
    say("captured steps: refused with adaptive capacity")
    m = Model(64, 16, 4, 512, 256, moe.Q_INT4_G32_F16, 2, seed=631, adaptive=dict(period=2, delta=2, pairs=1, floor=8))
    try:
        with pytest.raises(moe.MoeError) as ei:
            m.cache.set_graph(True)
        assert ei.value.code == moe.ERR_UNSUPPORTED
        m.cache.set_graph(False)
    finally:
        m.close()


def test_captured_steps_against_oracle():
    """The 48-layer Qwen3-30B-A3B shape with every expert resident (K = E): 32-token warm-up
    calls, then one-token captured steps that write every layer's input from inside the
    graph.  Every call is checked teacher-forced against the oracle (routing, plan records,
    slots), and every layer output of the captured steps within 2e-3 max|ref|."""
    from gpu_harness import check_stack_step
    L, H = 48, 2048
    say("captured steps vs oracle: L=48 E=128 k=8 H=2048 I=768 int4 K=E, layer inputs captured in the graph")
    m = Model(128, 128, 8, H, 768, moe.Q_INT4_G32_F16, L, n_distinct=131, seed=641, prefetch=True)
    try:
        m.cache.set_graph(True)
        sim = m.oracle_sim()
        rp = [m.router[l].data_ptr() for l in range(L)]
        step = 0
        xw = synth.ar1_streams(642, 32, 40, H)
        cap = torch.empty(L, 32, H, device="cuda")
        while not _all_resident(m):
            assert step < xw.shape[0], "warm-up did not make every expert resident"
            x = torch.from_numpy(xw[step]).cuda()
            out = torch.empty_like(x)
            n0 = len(m.records)
            m.cache.stack_forward(x, 32, rp, out, layer_inputs=cap)
            torch.cuda.synchronize()
            check_stack_step(m, sim, step, cap.cpu().numpy(), out.cpu().numpy(), m.records[n0:],
                             check_y=lambda s, l: False)
            step += 1
        n_warm = step
        cap1 = torch.empty(L, 1, H, device="cuda")
        out1 = torch.empty(1, H, device="cuda")
        worst, n_y = 0.0, 0
        for s in range(6):
            x = torch.from_numpy(synth.ar1_streams(650 + s, 1, 1, H)[0]).cuda()
            n0 = len(m.records)
            m.cache.stack_forward(x, 1, rp, out1, layer_inputs=cap1)
            torch.cuda.synchronize()
            st = m.cache.stats()                   # applies the captured step's plans (records)
            assert st["graph_steps"] == s + 1
            _near, w, ny = check_stack_step(m, sim, step, cap1.cpu().numpy(), out1.cpu().numpy(), m.records[n0:])
            worst, n_y = max(worst, w), n_y + ny
            step += 1
        assert n_y == 6 * L
        say(f"  {n_warm} warm-up calls, 6 captured steps, {n_y} layer outputs, worst max|err|/max|ref| = {worst:.2e}")
    finally:
        m.close()

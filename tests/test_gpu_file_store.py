"""Two-tier store (moe_cache_set_file_store) through the C ABI.

Expert blocks are read from a file into an LRU of pinned RAM blocks and uploaded
from there.  Against the same cache on the pinned host store: outputs bitwise
equal and the same plan records, for decode calls of several sizes and prefill
calls; without speculation the RAM counters equal the oracle's RAM tier replayed
over the same plans (with speculation, staged fills skip the tier, so only the
outputs are compared).
"""
import os
import sys
import tempfile

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
    # E, K, k, H, I, quant, L, flags, shared_expert, ram_blocks
    "int4": (64, 16, 4, 512, 256, moe.Q_INT4_G32_F16, 3, 0, False, 40),
    "e2m1-shared-pool": (64, 48, 4, 512, 256, moe.Q_E2M1_E4M3_G16, 3, moe.POOL_SHARED, True, 48),
    "f32": (16, 8, 2, 256, 128, moe.Q_F32, 3, 0, False, 32),
}

# decode calls of these token counts through every layer, with a prefill call of 40 tokens
# on layer 1 after the fourth
SCHED = [1, 1, 2, 4, 1, 8, 1, 3, 1, 1]


def _write_store(m, path):
    with open(path, "wb") as f:
        for l in range(m.L):
            for e in range(m.E):
                f.write(m.blocks[int(m.block_of[l, e])].tobytes())


def _run(case, file_path, prefetch, readers=3):
    E, K, k, H, I, quant, L, flags, shx, R = CASES[case]
    m = Model(E, K, k, H, I, quant, L, flags=flags, seed=711, shared_expert=shx, prefetch=prefetch)
    try:
        if file_path is not None:
            if not os.path.exists(file_path):
                _write_store(m, file_path)
            m.cache.set_file_store(file_path, R, readers)
        outs, calls = [], []
        for s, b in enumerate(SCHED):
            x = torch.from_numpy(synth.ar1_streams(720 + s, b, 1, H)[0]).cuda()
            for layer in range(L):
                n0 = len(m.records)
                x = m.forward(layer, x, residual=True, prefetch=prefetch)
                torch.cuda.synchronize()
                outs.append(x.cpu().numpy())
                ids = np.concatenate([np.array(r["ids"]) for r in m.records[n0:]]).reshape(-1, k)
                calls.append(("decode", layer, ids))
            if s == 3:
                xp = torch.from_numpy(synth.prefill_prompt(730, 40, H)).cuda()
                out = m.forward(1, xp, residual=True)
                torch.cuda.synchronize()
                outs.append(out.cpu().numpy())
                ids, _gate = m.cache.last_routing(40)
                calls.append(("prefill", 1, ids.copy()))
        st = m.cache.stats()
        return dict(outs=outs, recs=[dict(r) for r in m.records], stats=st, calls=calls, sim=m.oracle_sim())
    finally:
        m.close()


@pytest.mark.parametrize("case", sorted(CASES))
def test_file_store_bitwise_equals_pinned_store(case):
    E, K, k, H, I, quant, L, flags, shx, R = CASES[case]
    say(f"file store vs pinned store: {case} E={E} K={K} k={k} H={H} I={I} L={L} RAM blocks {R}")
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "experts.bin")
        for prefetch in (False, True):
            a = _run(case, None, prefetch)
            f = _run(case, path, prefetch)
            assert len(a["outs"]) == len(f["outs"])
            for i, (x, y) in enumerate(zip(a["outs"], f["outs"])):
                assert np.array_equal(x, y), (case, prefetch, i, float(np.max(np.abs(x - y))))
            assert a["recs"] == f["recs"], (case, prefetch)
            st = f["stats"]
            S = moe.expert_bytes(quant, H, I)
            assert st["bytes_read_file"] == st["ram_misses"] * S
            assert a["stats"]["ram_misses"] == 0 and a["stats"]["bytes_read_file"] == 0
            if prefetch:
                say(f"  prefetch on: RAM hits {st['ram_hits']} misses {st['ram_misses']}, "
                    f"{st['prefetch_used']} staged fills")
                continue
            # the RAM tier replayed by the oracle over the same plans
            sim = lru_sim(f["sim"], R)
            for kind, layer, ids in f["calls"]:
                if kind == "decode":
                    sim.decode(layer, ids)
                else:
                    sim.prefill(layer, ids)
            got = (st["ram_hits"], st["ram_misses"], st["ram_evictions"])
            want = (sim.ram.hits, sim.ram.misses, sim.ram.evictions)
            assert got == want, (case, got, want)
            assert st["ram_evictions"] > 0, case
            say(f"  RAM hits {got[0]} misses {got[1]} evictions {got[2]} (oracle {want})")


def lru_sim(sim, R):
    """A fresh oracle cache with the same pools and a RAM tier of R blocks."""
    from oracle import lru
    return lru.CacheSim(sim.E, sim.K, sim.k, sim.L, shared_pool=sim.shared, block_bytes=sim.block_bytes,
                        wave_rule=sim.wave_rule, ram_blocks=R)


def test_file_store_errors():
    say("file store: argument and file errors")
    m = Model(16, 8, 2, 256, 128, moe.Q_F32, 2, seed=741)
    try:
        with tempfile.TemporaryDirectory() as d:
            path = os.path.join(d, "short.bin")
            with open(path, "wb") as f:
                f.write(b"\0" * (m.S * 16 * 2 - 1))               # one byte short of 2 layers x 16 blocks
            with pytest.raises(moe.MoeError) as ei:
                m.cache.set_file_store(path, 32, 2)
            assert ei.value.code == moe.ERR_INVALID
            with pytest.raises(moe.MoeError) as ei:
                m.cache.set_file_store(os.path.join(d, "missing.bin"), 32, 2)
            assert ei.value.code == moe.ERR_IO
            with open(path, "ab") as f:
                f.write(b"\0")
            with pytest.raises(moe.MoeError) as ei:
                m.cache.set_file_store(path, 31, 2)                # below one prefill batch
            assert ei.value.code == moe.ERR_INVALID
            m.cache.set_file_store(path, 32, 2)
            with pytest.raises(moe.MoeError):
                m.cache.set_file_store(path, 32, 2)                # a second file store
            with pytest.raises(moe.MoeError):
                m.cache.set_layer(0, m.store.ptr)                  # host stores are refused now
    finally:
        m.close()


def test_file_store_with_captured_steps():
    """Once every expert is resident, one-token stack steps replay as graphs on a file-backed
    cache too: outputs bitwise equal to the pinned store's, RAM counters the oracle's."""
    E, K, k, H, I, L, R = 64, 64, 4, 512, 256, 3, 64
    say(f"file store + captured steps: int4 E={E} K={K} k={k} H={H} I={I} L={L}, RAM blocks {R}")
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "experts.bin")
        res = []
        for use_file in (False, True):
            m = Model(E, K, k, H, I, moe.Q_INT4_G32_F16, L, seed=751)
            try:
                if use_file:
                    _write_store(m, path)
                    m.cache.set_file_store(path, R, 2)
                m.cache.set_graph(True)
                rp = [m.router[l].data_ptr() for l in range(L)]
                xw = synth.ar1_streams(752, 32, 40, H)
                warm = 0
                while not all(m.cache.slot_of(l, e) >= 0 for l in range(L) for e in range(E)):
                    assert warm < xw.shape[0]
                    x = torch.from_numpy(xw[warm]).cuda()
                    m.cache.stack_forward(x, 32, rp, torch.empty_like(x))
                    torch.cuda.synchronize()
                    warm += 1
                out = torch.empty(1, H, device="cuda")
                outs = []
                for s in range(8):
                    x = torch.from_numpy(synth.ar1_streams(760 + s, 1, 1, H)[0]).cuda()
                    m.cache.stack_forward(x, 1, rp, out)
                    torch.cuda.synchronize()
                    outs.append(out.cpu().numpy().copy())
                st = m.cache.stats()
                recs = [dict(r) for r in m.records]
                res.append((outs, recs, st))
            finally:
                m.close()
    (o0, r0, s0), (o1, r1, s1) = res
    assert s0["graph_steps"] == 8 and s1["graph_steps"] == 8
    for a, b in zip(o0, o1):
        assert np.array_equal(a, b)
    assert r0 == r1
    from oracle import lru
    sim = lru.CacheSim(E, K, k, L, ram_blocks=R)
    for call in _group(r1):
        sim.decode(call[0]["layer"], np.concatenate([np.array(r["ids"]) for r in call]).reshape(-1, k))
    assert (s1["ram_hits"], s1["ram_misses"], s1["ram_evictions"]) == (sim.ram.hits, sim.ram.misses,
                                                                      sim.ram.evictions)
    say(f"  RAM hits {s1['ram_hits']} misses {s1['ram_misses']} evictions {s1['ram_evictions']}")


def _group(recs):
    """Plan records grouped into calls (t0 restarts at 0 with each call)."""
    calls = []
    for r in recs:
        if r["t0"] == 0:
            calls.append([])
        calls[-1].append(r)
    return calls


def test_file_store_adaptive_capacity_b32():
    """Adaptive per-layer capacity lets a layer hold up to E slots, so a wave may upload more
    than K blocks: the RAM tier must hold min(E, 32 * top_k) blocks (a smaller one is
    refused), and 32-token calls on a file-backed cache then match the pinned store bitwise
    (outputs and plan records) while a layer whose capacity grew uploads more than K blocks
    in one wave."""
    E, K, k, H, I, L = 128, 16, 8, 512, 256, 3
    ad = dict(period=2, delta=8, pairs=1, floor=8)
    need = max(32, min(max(K, E), 32 * k))
    sched = [1, 1, 1, 1, 1, 1, 32, 32, 1, 1, 32, 32, 32]
    say(f"file store + adaptive capacity: int4 E={E} K={K}/layer k={k} H={H} I={I} L={L}, calls of {sched} tokens, "
        f"RAM blocks {need}")
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "experts.bin")
        res = []
        for use_file in (False, True):
            m = Model(E, K, k, H, I, moe.Q_INT4_G32_F16, L, seed=771, adaptive=ad, prefetch=True)
            try:
                if use_file:
                    _write_store(m, path)
                    with pytest.raises(moe.MoeError) as ei:
                        m.cache.set_file_store(path, need - 1, 2)
                    assert ei.value.code == moe.ERR_INVALID
                    m.cache.set_file_store(path, need, 2)
                outs = []
                for s, b in enumerate(sched):
                    x = torch.from_numpy(synth.ar1_streams(772 + s, b, 1, H)[0]).cuda()
                    for layer in range(L):
                        x = m.forward(layer, x, residual=True, prefetch=True)
                    torch.cuda.synchronize()
                    outs.append(x.cpu().numpy())
                caps = [m.cache.layer_capacity(l) for l in range(L)]
                res.append((outs, [dict(r) for r in m.records], m.cache.stats(), caps))
            finally:
                m.close()
    (o0, r0, s0, c0), (o1, r1, s1, c1) = res
    for i, (a, b) in enumerate(zip(o0, o1)):
        assert np.array_equal(a, b), i
    assert r0 == r1 and c0 == c1
    most = max(len(r["fills"]) for r in r1)
    assert most > K, most                                     # a wave uploaded more than K blocks
    assert s1["ram_misses"] > 0 and s1["bytes_read_file"] == s1["ram_misses"] * moe.expert_bytes(
        moe.Q_INT4_G32_F16, H, I)
    say(f"  most fills in one wave {most}, capacities {c1}, RAM hits {s1['ram_hits']} misses {s1['ram_misses']} "
        f"evictions {s1['ram_evictions']}")

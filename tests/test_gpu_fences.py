"""Fence and failure-path checks of the upload paths through the C ABI (SGLang page, "Can
paging change the model's outputs?": paging bugs give fluent wrong outputs, not crashes).

* Poisoned, delayed uploads: with MOE_DEBUG_POISON every block an upload is about to
  overwrite is first filled with all-one bytes (NaN scales) on the upload's stream, and with
  MOE_DEBUG_DELAY_US a waiting kernel goes ahead of every upload.  A kernel that read a slot,
  a staging block or the prefill arena without waiting for its upload would read NaN or a
  stale expert; outputs and traces must stay bitwise those of a cache without the checks,
  and match the oracle.
* A failed upload submission (moe_debug_fail_upload): the call returns MOE_ERR_HIP, the
  wave's fills are rolled back (their experts not resident), and the next call uploads them
  again and matches the oracle.
* A router selection that stops waiting for the other workgroups' logits (forced with
  MOE_DEBUG_ROUTER_WAIT_US=0) is reported, and poisons only its own cache.
"""
import os
import sys

import numpy as np
import pytest
import torch

import expert_offload_lru_amd as moe
import synth
from gpu_harness import Model, check_routing, compare_records, tol_ok

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # E, K, k, H, I, quant, L, flags, n_distinct, shared_expert
    "int4-per-layer": (128, 24, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, 0, 131, False),
    "e2m1-shared-pool": (64, 48, 4, 512, 256, moe.Q_E2M1_E4M3_G16, 3, moe.POOL_SHARED, None, True),
}


def _run(case, checks):
    E, K, k, H, I, quant, L, flags, nd, shx = CASES[case]
    env = {"MOE_DEBUG_POISON": "1", "MOE_DEBUG_DELAY_US": "150"} if checks else {}
    os.environ.update(env)
    try:
        m = Model(E, K, k, H, I, quant, L, flags=flags, n_distinct=nd, seed=901, shared_expert=shx, prefetch=True)
    finally:
        for v in env:
            os.environ.pop(v, None)
    sim = m.oracle_sim()
    outs, worst = [], 0.0
    try:
        sched = [1] * 5 + [4] * 2 + [1] * 3
        for step, b in enumerate(sched):
            x = torch.from_numpy(synth.ar1_streams(902 + step, b, 1, H)[0]).cuda()
            for layer in range(L):
                n0 = len(m.records)
                out = m.forward(layer, x, residual=True, prefetch=True)
                torch.cuda.synchronize()
                x_np = x.cpu().numpy()
                recs = m.records[n0:]
                ids, gate, _ = check_routing(m, layer, x_np, np.concatenate([np.array(r["ids"]) for r in recs]),
                                             np.concatenate([np.array(r["gate"]) for r in recs]))
                _slots, orecs = sim.decode(layer, ids, step)
                compare_records(orecs, recs, where=(case, step, layer))
                o = out.cpu().numpy()
                ok, err, scale = tol_ok(o.astype(np.float64) - x_np, m.oracle_y(layer, x_np, ids, gate))
                worst = max(worst, err / scale)
                assert ok, (case, step, layer, err, scale)
                outs.append(o)
                x = out
            if step == 4:                       # a prefill call: uploads through the arena
                xp = torch.from_numpy(synth.prefill_prompt(950, 48, H)).cuda()
                out = m.forward(1, xp, residual=True, prefetch=False)
                torch.cuda.synchronize()
                outs.append(out.cpu().numpy())
        st = m.cache.stats()
        return outs, [dict(r) for r in m.records], st, worst
    finally:
        m.close()


@pytest.mark.parametrize("case", sorted(CASES))
def test_poisoned_delayed_uploads_change_nothing(case):
    say(f"fence checks: poisoned and delayed uploads vs plain uploads, {case}")
    o1, r1, s1, w1 = _run(case, True)
    o0, r0, s0, _w0 = _run(case, False)
    assert len(o1) == len(o0)
    for i, (a, b) in enumerate(zip(o1, o0)):
        assert np.all(np.isfinite(a)), (case, i)
        assert np.array_equal(a, b), (case, i, float(np.nanmax(np.abs(a - b))))
    assert r1 == r0
    assert s1["small"]["misses"] > 0 and s1["prefill"]["misses"] > 0
    say(f"  {len(o1)} outputs bitwise equal, worst max|err|/max|ref| {w1:.2e}, "
        f"{s1['prefetch_used']} staged fills, {s1['small']['misses'] + s1['large']['misses']} uploads")


def test_failed_upload_rolls_back_and_uploads_again():
    E, K, k, H, I, L = 64, 16, 4, 512, 256, 2
    say(f"failed upload submission: int4 E={E} K={K} k={k} H={H} I={I} L={L}, no speculation")
    m = Model(E, K, k, H, I, moe.Q_INT4_G32_F16, L, seed=911, prefetch=False)
    try:
        for step in range(4):                                  # fill the pools
            x = torch.from_numpy(synth.ar1_streams(912 + step, 4, 1, H)[0]).cuda()
            for layer in range(L):
                x = m.forward(layer, x, residual=True, prefetch=False)
        torch.cuda.synchronize()
        x = torch.from_numpy(synth.ar1_streams(920, 4, 1, H)[0]).cuda()   # new streams: misses
        x_np = x.cpu().numpy()
        ids, gate, _z, _p = m.oracle_route(0, x_np)
        wanted = list(dict.fromkeys(int(e) for e in ids.reshape(-1)))
        before = {e: m.cache.slot_of(0, e) for e in range(E)}
        misses = [e for e in wanted if before[e] < 0]
        assert misses, "the call needs uploads"
        n_rec = len(m.records)
        m.cache.debug_fail_upload(0)
        out = torch.empty_like(x)
        rc = m.cache.forward_rc(0, x, 4, m.router[0], out, flags=moe.FWD_RESIDUAL)
        torch.cuda.synchronize()
        assert rc == moe.ERR_HIP, rc
        assert len(m.records) == n_rec                         # no plan was recorded
        after = {e: m.cache.slot_of(0, e) for e in range(E)}
        assert all(after[e] < 0 for e in misses)               # the wave's fills rolled back
        assert all(after[e] == before[e] for e in wanted if before[e] >= 0)   # its hits stay
        freed = [s for s in range(K) if s not in set(v for v in after.values() if v >= 0)]
        assert len(freed) >= len(misses)                      # the filled slots are empty now
        # the same call again: the rolled-back experts are uploaded this time, and the layer
        # output is the oracle's
        out = m.forward(0, x, residual=True, prefetch=False)
        torch.cuda.synchronize()
        rec = m.records[-1]
        assert sorted(e for e, _s in rec["fills"]) == sorted(misses)
        gids, ggate, _ = check_routing(m, 0, x_np, np.array(rec["ids"]), np.array(rec["gate"]))
        ok, err, scale = tol_ok(out.cpu().numpy().astype(np.float64) - x_np, m.oracle_y(0, x_np, gids, ggate))
        assert ok, (err, scale)
        assert all(m.cache.slot_of(0, e) >= 0 for e in wanted)
        say(f"  {len(misses)} fills rolled back and uploaded again; max|err|/max|ref| {err / scale:.2e}")
        with pytest.raises(moe.MoeError):
            m.cache.debug_fail_upload(-2)
    finally:
        m.close()


def test_router_selection_that_stops_waiting_is_reported(monkeypatch):
    """The one-launch router's selecting workgroups wait for the other workgroups' logits for
    a bounded time.  With MOE_DEBUG_ROUTER_WAIT_US=0 every selection gives up at once:
    the call returns MOE_ERR_HIP (no routing was written), later forward calls of that cache
    refuse with MOE_ERR_HIP too, and a cache created without the setting is unaffected."""
    E, K, k, H, I, L = 64, 16, 4, 512, 256, 2
    say(f"router selection timeout: int4 E={E} K={K} k={k} H={H} I={I} L={L}")
    monkeypatch.setenv("MOE_DEBUG_ROUTER_WAIT_US", "0")
    m = Model(E, K, k, H, I, moe.Q_INT4_G32_F16, L, seed=931, prefetch=False)
    monkeypatch.delenv("MOE_DEBUG_ROUTER_WAIT_US")
    try:
        x = torch.from_numpy(synth.ar1_streams(932, 1, 1, H)[0]).cuda()
        out = torch.empty_like(x)
        rc = m.cache.forward_rc(0, x, 1, m.router[0], out, flags=moe.FWD_RESIDUAL)
        torch.cuda.synchronize()
        assert rc == moe.ERR_HIP, rc
        x8 = torch.from_numpy(synth.ar1_streams(933, 8, 1, H)[0]).cuda()   # the two-launch router
        rc = m.cache.forward_rc(0, x8, 8, m.router[0], torch.empty_like(x8), flags=moe.FWD_RESIDUAL)
        torch.cuda.synchronize()
        assert rc == moe.ERR_HIP, rc
        assert "stopped waiting" in moe.gpu_lib().moe_last_error().decode()
    finally:
        m.close()
    m = Model(E, K, k, H, I, moe.Q_INT4_G32_F16, L, seed=931, prefetch=False)
    try:
        x_np = synth.ar1_streams(932, 1, 1, H)[0]
        out = m.forward(0, torch.from_numpy(x_np).cuda(), residual=True, prefetch=False)
        torch.cuda.synchronize()
        rec = m.records[-1]
        gids, ggate, _ = check_routing(m, 0, x_np, np.array(rec["ids"]), np.array(rec["gate"]))
        ok, err, scale = tol_ok(out.cpu().numpy().astype(np.float64) - x_np, m.oracle_y(0, x_np, gids, ggate))
        assert ok, (err, scale)
    finally:
        m.close()

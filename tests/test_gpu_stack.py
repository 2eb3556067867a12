"""The native layer loop (moe_stack_forward) at one token, the call the decode
throughput is measured on, checked against the oracle layer by layer.

At one token the loop launches each layer's router and the early gate/up of its
resident picks behind the previous layer's down + combine, speculates up to five
layers ahead into the staging bank and reads staged fills through the GEMV.  Its
layer_inputs argument captures every layer's input, so each layer is checked
teacher-forced: routing against the oracle's on that input, the plan records and
slots against the oracle's LRU, the layer output within 2e-3 max|ref|.
"""
import sys

import numpy as np
import pytest
import torch

import expert_offload_lru_amd as moe
import synth
from gpu_harness import Model, check_stack_step

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_checked_stack(m, x0, check_y=lambda s, l: True, sim=None, first_step=0):
    """Stack calls of x0 [steps, b, H] with layer inputs captured, each checked against the
    oracle (continuing `sim` from step `first_step` when given).  Returns the oracle's cache
    simulation."""
    sim = sim or m.oracle_sim()
    rp = [m.router[l].data_ptr() for l in range(m.L)]
    sp = [m.shared[l].data_ptr() for l in range(m.L)] if m.shared is not None else None
    near = n_y = 0
    worst = 0.0
    b = x0.shape[1]
    cap = torch.empty(m.L, b, m.H, device="cuda")
    for i in range(x0.shape[0]):
        step = first_step + i
        x = torch.from_numpy(x0[i]).cuda()
        out = torch.empty_like(x)
        n0 = len(m.records)
        m.cache.stack_forward(x, b, rp, out, shared_ptrs=sp, layer_inputs=cap)
        torch.cuda.synchronize()
        nr, w, ny = check_stack_step(m, sim, step, cap.cpu().numpy(), out.cpu().numpy(), m.records[n0:], check_y)
        near, worst, n_y = near + nr, max(worst, w), n_y + ny
    say(f"  {x0.shape[0]} steps, {n_y} layer outputs checked, worst max|err|/max|ref| = {worst:.2e}, "
        f"near-tie deviations {near}")
    return sim


def test_stack_b1_qwen3_30b_full_size_against_oracle():
    """The measured configuration: 48 layers, E=128, top_k=8, int4 group-32, K=92 per layer,
    one token, speculation five layers ahead with a copy-queue limit of 4, early gate/up on.
    Two 32-token calls first fill every pool, so the one-token steps evict."""
    steps = 12
    say(f"stack b=1 vs oracle: L=48 E=128 k=8 H=2048 I=768 int4 K=92, prefetch 5 ahead, 2 filling 32-token "
        f"calls, then {steps} one-token steps, every layer output of those checked")
    m = Model(128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 48, n_distinct=131, seed=701, prefetch=True)
    try:
        m.cache.set_prefetch(4, 5)
        sim = run_checked_stack(m, synth.ar1_streams(703, 32, 2, 2048), check_y=lambda s, l: l % 12 == 0)
        assert all(sum(m.cache.slot_of(l, e) >= 0 for e in range(128)) == 92 for l in range(48))   # pools full
        m.cache.reset_stats()
        sim.stats = type(sim.stats)()                             # counters of the one-token steps only
        m.cache.set_timing(moe.TIME_GATE_UP_EARLY | moe.TIME_DOWN_EARLY | moe.TIME_DOWN, stride=1)
        sim = run_checked_stack(m, synth.ar1_streams(702, 1, steps, 2048), sim=sim, first_step=2)
        st = m.cache.stats()
        tm = m.cache.timing()
        o = sim.stats.b["small"]
        assert (st["small"]["hits"], st["small"]["misses"], st["small"]["evictions"]) == (o["hits"], o["misses"],
                                                                                         o["evictions"])
        assert st["small"]["evictions"] > 0                       # the pools churned
        assert st["prefetch_used"] > 0                            # staged fills were read through the GEMV
        assert tm["gate_up_early"]["launches"] == steps * 48      # one early gate/up per layer call
        # an early down + combine where the previous layer's speculative ids for the layer
        # showed every pick resident; layers whose plan then changed nothing were complete
        # after the early launches, and the host launched a down + combine for the others
        assert 0 < tm["down_early"]["launches"] <= steps * 48 and tm["down_early"]["bytes"] > 0
        assert 0 < tm["down"]["launches"] < steps * 48
        say(f"  prefetch issued/used/wasted {st['prefetch_issued']}/{st['prefetch_used']}/{st['prefetch_wasted']}, "
            f"hits {st['small']['hits']} misses {st['small']['misses']}; early down launches "
            f"{tm['down_early']['launches']}, layers completed by the early launches "
            f"{steps * 48 - tm['down']['launches']} of {steps * 48}")
    finally:
        m.close()


def test_stack_b1_flash_next_full_size_against_oracle():
    """The e2m1 shape: 48 layers, E=512 + shared expert, top_k=10, H=3072, I=512, one shared
    pool of 2048 slots, one token, speculation one layer ahead."""
    steps = 4
    say(f"stack b=1 vs oracle: L=48 E=512 k=10 H=3072 I=512 e2m1, shared pool 2048, shared expert, "
        f"{steps} steps, every layer output checked")
    m = Model(512, 2048, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 48, flags=moe.POOL_SHARED, n_distinct=131, seed=711,
              shared_expert=True, prefetch=True)
    try:
        m.cache.set_prefetch(4, 1)
        run_checked_stack(m, synth.ar1_streams(712, 1, steps, 3072))
        st = m.cache.stats()
        assert st["small"]["hits"] > 0 and st["prefetch_used"] > 0
    finally:
        m.close()


@pytest.mark.parametrize("b", [4, 32])
def test_stack_batched_against_oracle(b):
    """Batched stack calls (no early launch; b=32 plans three waves per layer)."""
    say(f"stack b={b} vs oracle: L=6 E=128 k=8 H=2048 I=768 int4 K=92, prefetch 3 ahead, 3 steps")
    m = Model(128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 6, n_distinct=131, seed=721 + b, prefetch=True)
    try:
        run_checked_stack(m, synth.ar1_streams(722 + b, b, 3, 2048))
        if b == 32:
            assert m.cache.stats()["large"]["plans"] == 3 * 6 * 3
    finally:
        m.close()

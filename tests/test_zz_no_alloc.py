"""moe_layer_forward_noalloc through the C ABI: the allocation-free decode call, whose
per-call device scratch is the library's static device array, against moe_layer_forward
on an identical cache (same kernels, so bitwise equal outputs and identical plan
records), over two calls in a row per layer, the second with fewer tokens; shapes whose
scratch exceeds the array and prefill-sized calls are refused."""
import sys

import numpy as np
import pytest
import torch

import expert_offload_lru_amd as moe
import synth
from gpu_harness import Model, compare_records

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = {
    # E, K, k, H, I, quant, L, flags, n_distinct, shared_expert, prefetch
    "int4-qwen3-shape": (128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 3, 0, 131, False, True),
    "e2m1-shared-pool-shared-expert": (512, 200, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 2, moe.POOL_SHARED, 131, True,
                                       True),
    "f32-churn": (16, 4, 2, 256, 128, moe.Q_F32, 2, 0, None, False, False),
}


def _run(case, noalloc):
    E, K, k, H, I, quant, L, flags, nd, shx, pf = CASES[case]
    m = Model(E, K, k, H, I, quant, L, flags=flags, n_distinct=nd, seed=801, shared_expert=shx, prefetch=pf)
    try:
        outs = []
        for s, b in enumerate([12, 1, 32, 4, 1]):       # each call after the first is smaller or larger
            x = torch.from_numpy(synth.ar1_streams(802 + s, b, 1, H)[0]).cuda()
            for layer in range(L):
                out = torch.empty_like(x)
                nxt = m.router[layer + 1] if (pf and layer + 1 < L) else None
                sw = m.shared[layer] if m.shared is not None else None
                call = m.cache.forward_noalloc if noalloc else m.cache.forward
                call(layer, x, b, m.router[layer], out, shared_w=sw, next_router_w=nxt, residual=True)
                torch.cuda.synchronize()
                outs.append(out.cpu().numpy())
                x = out
        return outs, [dict(r) for r in m.records], m.cache.stats()
    finally:
        m.close()


@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_equals_layer_forward(case):
    say(f"allocation-free decode call vs moe_layer_forward: {case}")
    o1, r1, s1 = _run(case, True)
    o0, r0, s0 = _run(case, False)
    assert len(o1) == len(o0)
    for i, (a, b) in enumerate(zip(o1, o0)):
        assert np.all(np.isfinite(a))
        assert np.array_equal(a, b), (case, i, float(np.max(np.abs(a - b))))
    compare_records(r0, r1, where=case)
    assert [r["ids"] for r in r1] == [r["ids"] for r in r0]
    assert s1["small"] == s0["small"] and s1["large"] == s0["large"]
    say(f"  {len(o1)} calls bitwise equal, {len(r1)} plan records equal")


def test_noalloc_two_calls_second_smaller():
    """Two calls in a row on one layer, 32 tokens then 3: the second reads nothing the
    first left in the array (outputs equal the regular call's bitwise)."""
    say("allocation-free decode call: 32 tokens then 3 on one layer")
    res = []
    for noalloc in (True, False):
        m = Model(64, 48, 4, 512, 256, moe.Q_INT4_G32_F16, 1, seed=811)
        try:
            outs = []
            for s, b in enumerate((32, 3)):
                x = torch.from_numpy(synth.ar1_streams(812 + s, b, 1, 512)[0]).cuda()
                out = torch.empty_like(x)
                (m.cache.forward_noalloc if noalloc else m.cache.forward)(0, x, b, m.router[0], out, residual=True)
                torch.cuda.synchronize()
                outs.append(out.cpu().numpy())
            res.append(outs)
        finally:
            m.close()
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


def test_noalloc_refusals():
    say("allocation-free decode call: prefill-sized calls and oversized shapes are refused")
    m = Model(16, 8, 2, 256, 128, moe.Q_F32, 1, seed=821)
    try:
        x = torch.zeros(33, 256, device="cuda")
        out = torch.empty_like(x)
        with pytest.raises(moe.MoeError) as ei:
            m.cache.forward_noalloc(0, x, 33, m.router[0], out)
        assert ei.value.code == moe.ERR_UNSUPPORTED
    finally:
        m.close()
    # top_k 16, hidden = inter = 8192: h and Y of 32 tokens x 17 pairs take 2 x 17.8 MB, more
    # than the 32 MiB array (refused before the layer's host store is looked at)
    c = moe.Cache(1024, 16, 16, 8192, 8192, moe.Q_INT4_G32_F16, 1, 0)
    try:
        x = torch.zeros(1, 8192, device="cuda")
        out = torch.empty_like(x)
        rw = torch.zeros(1024, 8192, device="cuda")
        with pytest.raises(moe.MoeError) as ei:
            c.forward_noalloc(0, x, 1, rw, out)
        assert ei.value.code == moe.ERR_UNSUPPORTED
    finally:
        c.close()

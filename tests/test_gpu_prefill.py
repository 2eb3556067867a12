"""GPU parity of the prefill path (> 32 tokens) through the C ABI against the oracle:
routing exact (up to near ties), outputs within 2e-3 max|ref|, LRU state unchanged,
cold and warm caches bitwise equal."""
import sys

import numpy as np
import pytest
import torch

import expert_offload_lru_amd as moe
import synth
from gpu_harness import Model, check_routing, tol_ok

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def residency(m):
    return [[m.cache.slot_of(l, e) for e in range(m.E)] for l in range(m.L)]


def prefill_and_check(m, layer, x_np, sample=None, residual=True):
    x = torch.from_numpy(x_np).cuda()
    out = m.forward(layer, x, residual=residual, prefetch=False)
    torch.cuda.synchronize()
    gids, ggate = m.cache.last_routing(x_np.shape[0])
    rows = np.arange(x_np.shape[0]) if sample is None else np.asarray(sample)
    ids, gate, _dev = check_routing(m, layer, x_np[rows], gids[rows], ggate[rows])
    y_gpu = out.cpu().numpy()[rows].astype(np.float64) - (x_np[rows].astype(np.float64) if residual else 0.0)
    y_ref = m.oracle_y(layer, x_np[rows], ids, gate)
    ok, err, scale = tol_ok(y_gpu, y_ref)
    say(f"  prefill layer {layer}: {x_np.shape[0]} tokens, max|err|/max|ref| = {err / scale:.2e}")
    assert ok, (err, scale)
    return out


def test_prefill_small_ragged_cold_and_warm():
    say("prefill: E=16 k=2 H=256 I=256 int4, K=8, 100 tokens, cold then partly warm")
    m = Model(16, 8, 2, 256, 256, moe.Q_INT4_G32_F16, 1, seed=111)
    x = synth.prefill_prompt(112, 100, 256)
    try:
        before = residency(m)
        out_cold = prefill_and_check(m, 0, x).cpu().numpy()
        assert residency(m) == before                      # LRU untouched
        st = m.cache.stats()["prefill"]
        assert st["hits"] == 0 and st["misses"] > 0 and st["plans"] == 1
        # warm some experts through decode calls (their routing checked too: the routing
        # buffers were regrown for the prefill call), then prefill again: same bits
        xs = synth.ar1_streams(113, 1, 6, 256)
        for s in range(6):
            m.forward(0, torch.from_numpy(xs[s]).cuda(), residual=True)
            torch.cuda.synchronize()
            gids, ggate = m.cache.last_routing(xs[s].shape[0])
            check_routing(m, 0, xs[s], gids, ggate)
        warm = residency(m)
        assert any(s >= 0 for s in warm[0])
        out_warm = prefill_and_check(m, 0, x).cpu().numpy()
        assert residency(m) == warm
        assert np.array_equal(out_cold, out_warm)
        st = m.cache.stats()["prefill"]
        assert st["hits"] > 0
    finally:
        m.close()


def test_prefill_e2m1_shared_expert():
    say("prefill: E=64 k=4 H=512 I=256 e2m1, shared expert, shared pool, 80 tokens")
    m = Model(64, 24, 4, 512, 256, moe.Q_E2M1_E4M3_G16, 2, flags=moe.POOL_SHARED, seed=121, shared_expert=True)
    x = synth.prefill_prompt(122, 80, 512)
    try:
        out = prefill_and_check(m, 0, x)
        prefill_and_check(m, 1, out.cpu().numpy())
    finally:
        m.close()


def test_prefill_many_tokens_per_expert_and_batches():
    say("prefill: E=40 k=4 H=256 I=256 int4, 700 tokens (2 expert batches, items > 64 rows)")
    m = Model(40, 10, 4, 256, 256, moe.Q_INT4_G32_F16, 1, seed=131)
    x = synth.prefill_prompt(132, 700, 256)
    try:
        prefill_and_check(m, 0, x)
        assert m.cache.stats()["prefill"]["misses"] > 32
    finally:
        m.close()


def test_prefill_full_qwen3_30b_shape_2048_tokens():
    say("prefill full size: 2048 tokens, E=128 k=8 H=2048 I=768 int4, K=92, 2 layers, every token checked")
    m = Model(128, 92, 8, 2048, 768, moe.Q_INT4_G32_F16, 2, n_distinct=131, seed=141)
    x = synth.prefill_prompt(142, 2048, 2048)
    try:
        out = prefill_and_check(m, 0, x)
        prefill_and_check(m, 1, out.cpu().numpy())
        st = m.cache.stats()["prefill"]
        assert st["plans"] == 2 and st["hits"] + st["misses"] == st["union_sum"]
    finally:
        m.close()


def test_prefill_f32_ragged_steps_and_column_tiles():
    say("prefill: E=16 k=2 H=192 I=384 fp32 weights, 90 tokens (3 and 6 reduction steps, a half column tile)")
    m = Model(16, 8, 2, 192, 384, moe.Q_F32, 1, seed=151)
    x = synth.prefill_prompt(152, 90, 192)
    try:
        prefill_and_check(m, 0, x)
    finally:
        m.close()


def test_prefill_partly_resident_many_upload_batches():
    say("prefill: E=100 k=4 H=256 I=768 int4, K=30 warmed by decode, 600 tokens (residents + 3 upload batches)")
    m = Model(100, 30, 4, 256, 768, moe.Q_INT4_G32_F16, 1, seed=161)
    x = synth.prefill_prompt(162, 600, 256)
    try:
        out_cold = prefill_and_check(m, 0, x).cpu().numpy()
        xs = synth.ar1_streams(163, 4, 12, 256)
        for s in range(12):
            m.forward(0, torch.from_numpy(xs[s]).cuda(), residual=True)
            torch.cuda.synchronize()
        warm = residency(m)
        assert sum(s >= 0 for s in warm[0]) == 30
        out_warm = prefill_and_check(m, 0, x).cpu().numpy()
        assert residency(m) == warm
        assert np.array_equal(out_cold, out_warm)
        st = m.cache.stats()["prefill"]
        assert st["plans"] == 2 and st["hits"] > 0 and st["misses"] > 2 * 32
    finally:
        m.close()


def test_prefill_router_tiles_ragged():
    say("prefill: E=18 k=3 H=256 I=256 int4, 33 and 49 tokens (router tiles of 16 tokens x 16 experts, ragged both ways)")
    m = Model(18, 6, 3, 256, 256, moe.Q_INT4_G32_F16, 1, seed=171)
    try:
        for n, seed in ((33, 172), (49, 173)):
            prefill_and_check(m, 0, synth.prefill_prompt(seed, n, 256))
    finally:
        m.close()


def test_prefill_flash_next_shape_thin_items():
    """The Flash-Next shape: 512 tokens spread over 512 experts (about ten rows each, so mostly
    one-row-tile items), a shared expert of all 512 rows, every touched expert uploaded through
    the arena in batches of 32; 96 sampled tokens of each layer checked against the oracle."""
    say("prefill: E=512 k=10 H=3072 I=512 e2m1, shared pool K=2048, shared expert, 512 tokens, 2 layers")
    m = Model(512, 2048, 10, 3072, 512, moe.Q_E2M1_E4M3_G16, 2, flags=moe.POOL_SHARED, n_distinct=131, seed=201,
              shared_expert=True)
    x = synth.prefill_prompt(202, 512, 3072)
    sample = np.random.default_rng(203).choice(512, 96, replace=False)
    try:
        out = prefill_and_check(m, 0, x, sample=sample)
        prefill_and_check(m, 1, out.cpu().numpy(), sample=sample)
        st = m.cache.stats()["prefill"]
        assert st["plans"] == 2 and st["hits"] == 0 and st["misses"] > 2 * 8 * 32
        assert st["hits"] + st["misses"] == st["union_sum"]
    finally:
        m.close()


def test_prefill_workspace_grows_and_shrinks():
    """One cache, prompts of 40, 700 and 90 tokens: the prefill workspace (the plan's staging in
    mapped host memory and its device copy, whose parts sit at offsets set by the capacity) is
    reallocated for the longer prompt and reused for the shorter one; every call checked."""
    say("prefill: E=40 k=4 H=256 I=256 int4, K=10, 40 then 700 then 90 tokens on one cache")
    m = Model(40, 10, 4, 256, 256, moe.Q_INT4_G32_F16, 1, seed=211)
    try:
        outs = {}
        for n, seed in ((40, 212), (700, 213), (90, 214)):
            x = synth.prefill_prompt(seed, n, 256)
            outs[n] = prefill_and_check(m, 0, x).cpu().numpy()
        # the short prompt again after the long one: same bits
        again = prefill_and_check(m, 0, synth.prefill_prompt(212, 40, 256)).cpu().numpy()
        assert np.array_equal(outs[40], again)
        assert m.cache.stats()["prefill"]["plans"] == 4
    finally:
        m.close()

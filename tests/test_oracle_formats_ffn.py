"""Pins of the oracle's number formats, dequantisation, FFN and layer (CPU)."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import ffn, formats, route


# ----------------------------------------------------------------------------- number formats

def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = formats.E4M3_TABLE
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3_spec_facts():
    t = formats.E4M3_TABLE
    assert np.nonzero(np.isnan(t))[0].tolist() == [0x7F, 0xFF]
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0
    assert t[1] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
    assert np.array_equal(np.diff(t[:0x7F]) > 0, np.ones(0x7E, bool))       # increasing over 0..126


def test_e2m1_table_is_the_ocp_value_set():
    # OCP Microscaling spec, FP4 E2M1: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert formats.E2M1_TABLE[:8].tolist() == mags
    assert formats.E2M1_TABLE[8:].tolist() == [-m for m in mags]


def test_hand_built_int4_matrix():
    # one row of 32 weights: byte j holds elements 2j (low) and 2j+1 (high)
    nib = np.zeros(16, dtype=np.uint8)
    nib[0] = 0x9A            # element 0 = 10 -> +2, element 1 = 9 -> +1
    nib[15] = 0x08 | 0xF0    # element 30 = 8 -> 0, element 31 = 15 -> +7
    nib[1:15] = 0x08 | 0x00  # even elements 0, odd elements 0 -> -8
    scale = np.array([0.5], dtype="<f2").view(np.uint8)
    w = formats.decode_matrix(formats.INT4_G32, np.concatenate([nib, scale]), 1, 32)[0]
    assert w[0] == 1.0 and w[1] == 0.5
    assert w[2] == 0.0 and w[3] == -4.0
    assert w[30] == 0.0 and w[31] == 3.5


def test_hand_built_e2m1_matrix():
    nib = np.zeros(8, dtype=np.uint8)
    nib[0] = 0x1 | (0xF << 4)       # element 0 = +0.5, element 1 = -6
    nib[7] = 0x5 | (0xA << 4)       # element 14 = +3,  element 15 = -1
    scale = np.array([0x40], dtype=np.uint8)   # E4M3 0x40: exponent 8 -> 2.0
    w = formats.decode_matrix(formats.E2M1_G16, np.concatenate([nib, scale]), 1, 16)[0]
    assert w[0] == 1.0 and w[1] == -12.0 and w[14] == 6.0 and w[15] == -2.0
    assert (w[2:14] == 0).all()


def test_generator_round_trip_on_representable_int4():
    rng = np.random.default_rng(0)
    q = rng.integers(-7, 8, size=(4, 64)).astype(np.float64)   # |q| <= 7 so amax = 7 s
    q[:, 0] = 7                                         # amax = 7 s exactly per group
    q[:, 32] = -7
    s = 2.0 ** -6
    w = (q * s).astype(np.float32)
    nib, sc = synth.quantize_int4_g32(w)
    raw = np.concatenate([nib.reshape(-1), sc.astype("<f2").view(np.uint8).reshape(-1)])
    assert np.array_equal(formats.decode_matrix(formats.INT4_G32, raw, 4, 64), w.astype(np.float64))


def test_generator_round_trip_on_representable_e2m1():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, size=(3, 32))
    codes[:, 0] = 7                                     # |value| 6 present in each group
    codes[:, 16] = 15
    s = formats.E4M3_TABLE[0x2A]                        # a normal E4M3 scale
    w = (formats.E2M1_TABLE[codes] * s).astype(np.float32)
    nib, sc = synth.quantize_e2m1_g16(w)
    raw = np.concatenate([nib.reshape(-1), sc.reshape(-1)])
    assert np.array_equal(formats.decode_matrix(formats.E2M1_G16, raw, 3, 32), w.astype(np.float64))


@pytest.mark.parametrize("quant", [0, 1, 2])
def test_block_size_and_decode_shapes(quant):
    H, I = 256, 256
    blk = synth.expert_block(5, 0, 1, quant, H, I)
    assert blk.size == formats.expert_bytes(quant, H, I) == synth.expert_bytes(quant, H, I)
    wg, wu, wd = formats.decode_expert(quant, blk, H, I)
    assert wg.shape == (I, H) and wu.shape == (I, H) and wd.shape == (H, I)
    for w in (wg, wu, wd):
        assert np.isfinite(w).all() and 0.01 < w.std() < 0.03


def test_expert_bytes_of_the_workloads():
    assert formats.expert_bytes(formats.F32, 256, 128) == 393216
    assert formats.expert_bytes(formats.INT4_G32, 2048, 768) == 2654208
    assert formats.expert_bytes(formats.E2M1_G16, 3072, 512) == 2654208


# ----------------------------------------------------------------------------- FFN and layer

def test_silu_special_values():
    assert ffn.silu(0.0) == 0.0
    assert abs(ffn.silu(40.0) - 40.0) < 1e-12
    assert abs(ffn.silu(-40.0)) < 1e-15
    assert abs(ffn.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


def test_hand_worked_ffn():
    # x = (1, -1): g = (1, -1), u = (0, -2), h = (0, 2/(1+e)), y = W_d h = (0, 2/(1+e))
    wg = np.array([[1.0, 0.0], [0.0, 1.0]])
    wu = np.array([[1.0, 1.0], [0.0, 2.0]])
    wd = np.array([[1.0, 0.0], [1.0, 1.0]])
    y = ffn.expert_ffn(np.array([1.0, -1.0]), wg, wu, wd)
    assert y[0] == 0.0 and abs(y[1] - 2.0 / (1.0 + math.e)) < 1e-15


def test_single_expert_layer_is_a_swiglu_mlp():
    rng = np.random.default_rng(3)
    H, I = 16, 24
    wg, wu, wd = (rng.standard_normal(s) * 0.3 for s in ((I, H), (I, H), (H, I)))
    x = rng.standard_normal((5, H))
    y, ids, gate = ffn.moe_layer(x, rng.standard_normal((1, H)), 1, lambda l, e: (wg, wu, wd))
    assert (ids == 0).all() and np.all(gate == 1.0)
    tx = torch.tensor(x)
    ref = (torch.nn.functional.silu(tx @ torch.tensor(wg).T) * (tx @ torch.tensor(wu).T)) @ torch.tensor(wd).T
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("with_shared", [False, True])
def test_dense_brute_force_equals_sparse(with_shared):
    rng = np.random.default_rng(4)
    E, k, H, I = 12, 3, 32, 16
    experts = [tuple(rng.standard_normal(s) * 0.2 for s in ((I, H), (I, H), (H, I))) for _ in range(E)]
    shared = tuple(rng.standard_normal(s) * 0.2 for s in ((I, H), (I, H), (H, I))) if with_shared else None
    w_r = rng.standard_normal((E, H))
    x = rng.standard_normal((6, H))
    y, _, _ = ffn.moe_layer(x, w_r, k, lambda l, e: experts[e], shared=shared)
    yd = ffn.moe_layer_dense(x, w_r, k, experts, shared=shared)
    assert np.max(np.abs(y - yd)) <= 1e-12 * np.max(np.abs(yd))


def test_hand_worked_four_expert_layer():
    # E = 4 scalar experts (H = I = 1): expert e is FFN(x) = d_e silu(g_e x) (u_e x)
    g = [1.0, 2.0, 0.0, 1.0]
    u = [1.0, 1.0, 5.0, -1.0]
    d = [1.0, 0.5, 1.0, 2.0]
    experts = lambda l, e: (np.array([[g[e]]]), np.array([[u[e]]]), np.array([[d[e]]]))
    w_r = np.array([[1.0], [2.0], [-1.0], [0.0]])     # x = 1: z = (1, 2, -1, 0) -> top-2 = (1, 0)
    y, ids, gate = ffn.moe_layer(np.array([[1.0]]), w_r, 2, experts)
    assert ids[0].tolist() == [1, 0]
    zsum = math.e + math.e ** 2 + math.e ** -1 + 1.0
    f1 = 0.5 * (2.0 / (1.0 + math.exp(-2.0))) * 1.0   # expert 1 at x = 1
    f0 = 1.0 * (1.0 / (1.0 + math.exp(-1.0))) * 1.0   # expert 0 at x = 1
    expect = (math.e ** 2 * f1 + math.e * f0) / zsum
    assert abs(y[0, 0] - expect) < 1e-15


def test_gate_not_renormalised():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 8))
    ids, gate, z, p = route.route(x, rng.standard_normal((10, 8)), 4)
    assert (gate.sum(axis=1) < 1.0).all()


# ----------------------------------------------------------------------------- layer for a given routing

def _random_layer(seed, E, H, I, shared):
    rng = np.random.default_rng(seed)
    experts = [tuple(rng.standard_normal(s) * 0.2 for s in ((I, H), (I, H), (H, I))) for _ in range(E)]
    sh = tuple(rng.standard_normal(s) * 0.2 for s in ((I, H), (I, H), (H, I))) if shared else None
    return rng, experts, sh


@pytest.mark.parametrize("with_shared", [False, True])
def test_given_routing_equals_layer_and_dense(with_shared):
    # fed the oracle's own routing, the checker every GPU test uses gives the per-token
    # sparse layer and the dense brute force over all E experts
    rng, experts, shared = _random_layer(6, 10, 24, 12, with_shared)
    w_r = rng.standard_normal((10, 24))
    x = rng.standard_normal((9, 24))
    y, ids, gate = ffn.moe_layer(x, w_r, 4, lambda l, e: experts[e], shared=shared)
    yg = ffn.moe_layer_given_routing(x, ids, gate, lambda l, e: experts[e], shared=shared)
    yd = ffn.moe_layer_dense(x, w_r, 4, experts, shared=shared)
    assert np.max(np.abs(yg - y)) <= 1e-13 * np.max(np.abs(y))
    assert np.max(np.abs(yg - yd)) <= 1e-12 * np.max(np.abs(yd))


def test_given_routing_hand_worked_gates_layers_and_shared():
    # scalar experts (H = I = 1): FFN_e(x) = d_e silu(g_e x) (u_e x); the gate of pick j
    # multiplies the expert of pick j, the experts come from the named layer, and the
    # shared expert enters with weight 1
    table = {0: [(1.0, 1.0, 1.0), (2.0, 1.0, 0.5), (0.0, 5.0, 1.0)],
             3: [(1.0, 2.0, 3.0), (1.0, -1.0, 2.0), (2.0, 2.0, 2.0)]}
    experts = lambda l, e: tuple(np.array([[v]]) for v in table[l][e])
    s = lambda z: z / (1.0 + math.exp(-z))
    x = np.array([[1.0], [2.0]])
    ids = np.array([[1, 0], [2, 1]])
    gate = np.array([[0.25, 0.5], [0.125, 0.75]])
    shared = tuple(np.array([[v]]) for v in (1.0, 1.0, -1.0))
    y = ffn.moe_layer_given_routing(x, ids, gate, experts, layer=3, shared=shared)
    f = lambda e, xv: table[3][e][2] * s(table[3][e][0] * xv) * (table[3][e][1] * xv)
    sh = lambda xv: -1.0 * s(xv) * xv
    expect0 = 0.25 * f(1, 1.0) + 0.5 * f(0, 1.0) + sh(1.0)
    expect1 = 0.125 * f(2, 2.0) + 0.75 * f(1, 2.0) + sh(2.0)
    assert abs(y[0, 0] - expect0) < 1e-15 and abs(y[1, 0] - expect1) < 1e-14
    # the same routing without the shared expert, and the other layer
    y0 = ffn.moe_layer_given_routing(x, ids, gate, experts, layer=0)
    g0 = lambda e, xv: table[0][e][2] * s(table[0][e][0] * xv) * (table[0][e][1] * xv)
    assert abs(y0[0, 0] - (0.25 * g0(1, 1.0) + 0.5 * g0(0, 1.0))) < 1e-15
    assert abs(y0[1, 0] - (0.125 * g0(2, 2.0) + 0.75 * g0(1, 2.0))) < 1e-15


def test_given_routing_grouped_rows_equal_one_pick_at_a_time():
    # many tokens sharing experts (the prefill case): per-expert row groups give the
    # one-vector-per-pick sum of the definition
    rng, experts, shared = _random_layer(7, 6, 16, 8, True)
    x = rng.standard_normal((40, 16))
    ids = np.stack([rng.permutation(6)[:3] for _ in range(40)])
    gate = rng.random((40, 3))
    y = ffn.moe_layer_given_routing(x, ids, gate, lambda l, e: experts[e], shared=shared)
    ref = np.zeros_like(x)
    for t in range(40):
        for j in range(3):
            ref[t] += gate[t, j] * ffn.expert_ffn(x[t], *experts[ids[t, j]])
        ref[t] += ffn.expert_ffn(x[t], *shared)
    assert np.max(np.abs(y - ref)) <= 1e-13 * np.max(np.abs(ref))

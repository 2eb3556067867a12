"""Pins of the oracle's router (CPU)."""
import math

import numpy as np

from oracle import route


def test_zero_input_gives_lowest_ids_and_uniform_gates():
    E, H, k = 16, 8, 3
    w = np.random.default_rng(0).standard_normal((E, H))
    ids, gate, z, p = route.route(np.zeros((2, H)), w, k)
    assert (z == 0).all()
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    assert np.allclose(gate, 1.0 / E, rtol=0, atol=1e-15)


def test_duplicated_rows_tie_to_lower_index():
    rng = np.random.default_rng(1)
    E, H = 8, 6
    w = rng.standard_normal((E, H)) * 0.1
    w[2] = 1.0
    w[5] = w[2]          # expert 5 duplicates expert 2
    w[7] = w[2]
    x = rng.standard_normal((1, H))
    # make expert 2 (and its copies) the clear winner: z = 3 H for them, |z| < 3 H otherwise
    x[0] = w[2] * 3
    ids, *_ = route.route(x, w, 3)
    assert ids[0].tolist() == [2, 5, 7]


def test_hand_worked_four_experts():
    # W_r rows pick x0, x1, x0+x1 and x3; x = (1, 2, 0, 3) -> z = (1, 2, 3, 3)
    w = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [1, 1, 0, 0], [0, 0, 0, 1]], dtype=np.float32)
    x = np.array([[1, 2, 0, 3]], dtype=np.float32)
    ids, gate, z, p = route.route(x, w, 2)
    assert z[0].tolist() == [1.0, 2.0, 3.0, 3.0]
    assert ids[0].tolist() == [2, 3]           # tie between 2 and 3 -> lower index first
    # gate of each pick: e^3 / (e + e^2 + 2 e^3) = 1 / (2 + e^-1 + e^-2)
    expect = 1.0 / (2.0 + math.exp(-1.0) + math.exp(-2.0))
    assert abs(gate[0, 0] - expect) < 1e-15 and abs(gate[0, 1] - expect) < 1e-15
    # top-1 of x = (0, 5, 1, 1): z = (0, 5, 5, 1) -> expert 1 (tie with 2, lower index)
    ids1, *_ = route.route(np.array([[0, 5, 1, 1]], dtype=np.float32), w, 1)
    assert ids1[0].tolist() == [1]


def test_rank_order_matches_python_sort_on_small_ties():
    rng = np.random.default_rng(2)
    for _ in range(200):
        E = int(rng.integers(2, 12))
        z = rng.integers(-3, 4, size=E).astype(np.float64)    # many exact ties
        expect = sorted(range(E), key=lambda e: (-z[e], e))
        assert route.rank_order(z).tolist() == expect


def test_softmax_sums_to_one_and_is_monotone():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((5, 128)) * 4
    p = route.softmax(z)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-14)
    for t in range(5):
        order = np.argsort(z[t])
        assert (np.diff(p[t][order]) >= 0).all()


def test_softmax_matches_scipy():
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(4)
    z = rng.standard_normal((3, 40)) * 10
    assert np.allclose(route.softmax(z), sp_softmax(z, axis=1), rtol=1e-13, atol=0)


def test_near_tie_detection_and_matching():
    w = np.eye(4)
    x = np.array([[1.0, 1.0 + 1e-13, 0.5, 0.0]])
    z = route.logits(x, w)
    a = route.abs_mass(x, w)
    ties = route.near_ties(z, a, 2)
    assert (0, 0) in ties                       # ranks 0 and 1 are 1e-13 apart
    ids, *_ = route.route(x, w, 2)
    assert ids[0].tolist() == [1, 0]
    assert route.ids_match_with_ties(ids, np.array([[0, 1]]), z, a)
    assert not route.ids_match_with_ties(ids, np.array([[1, 2]]), z, a)

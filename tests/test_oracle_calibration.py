"""Pins for the oracle's offline anchor selection: eq. sim, eq. w and the DP."""
import math

import numpy as np
import pytest

import oracle
from long_context_anchor_amd import synth


def test_sim_self_is_one_and_bounded():
    r = np.random.default_rng(0)
    for _ in range(20):
        n = int(r.integers(2, 60))
        k = int(r.integers(1, n + 1))
        pa = r.dirichlet(np.ones(n))
        pb = r.dirichlet(np.ones(n))
        assert abs(oracle.sim(pa, pa, k) - 1.0) < 1e-15
        s = oracle.sim(pa, pb, k)
        assert 0.0 <= s <= 1.0 + 1e-15


def test_sim_denominator_is_best_k_subset_mass():
    # sim(a,b) * best mass = mass of a's set, with best mass from brute force
    import itertools
    r = np.random.default_rng(1)
    for n in range(2, 9):
        pa, pb = r.dirichlet(np.ones(n)), r.dirichlet(np.ones(n))
        for k in range(1, n + 1):
            best = max(pb[list(c)].sum() for c in itertools.combinations(range(n), k))
            Ia = oracle.topk_full_sort(pa, k)
            assert abs(oracle.sim(pa, pb, k) - pb[Ia].sum() / best) < 1e-13


def test_sim_same_topk_set_gives_one():
    pa = np.array([0.5, 0.3, 0.1, 0.1])
    pb = np.array([0.35, 0.45, 0.1, 0.1])
    assert abs(oracle.sim(pa, pb, 2) - 1.0) < 1e-15
    assert abs(oracle.sim(pa, pb, 1) - 0.35 / 0.45) < 1e-15


def test_layer_weight_closed_forms():
    x = np.random.default_rng(2).standard_normal((5, 16))
    assert abs(oracle.layer_weight(x, x)) < 1e-14
    assert abs(oracle.layer_weight(x, -x) - 2.0) < 1e-14
    assert abs(oracle.layer_weight(x, 3.5 * x)) < 1e-14
    e = np.eye(4)
    assert abs(oracle.layer_weight(e[:2], e[2:]) - 1.0) < 1e-15
    with pytest.raises(ValueError):
        oracle.layer_weight(np.zeros((1, 4)), e[:1])


def test_weighted_similarity_layout():
    sb = np.arange(16, dtype=float).reshape(4, 4)
    w = np.array([1.0, 2.0, 3.0, 4.0])
    S = oracle.weighted_similarity(sb, w)
    assert S[1, 3] == 4.0 * 7.0 and S[3, 1] == 0.0 and S[2, 2] == 3.0 * 10.0


def test_dp_matches_brute_force():
    r = np.random.default_rng(3)
    for L in range(1, 11):
        for M in range(1, L + 1):
            for trial in range(3):
                S = np.triu(r.random((L, L)))
                np.fill_diagonal(S, 1.0 + r.random(L))
                anchors, val = oracle.dp_select_anchors(S, M)
                bset, bval = oracle.brute_force_anchors(S, M)
                assert abs(val - bval) < 1e-12
                assert abs(oracle.coverage_score(S, anchors) - val) < 1e-12
                assert anchors[0] == 0 and len(anchors) == M
                assert anchors == sorted(set(anchors))


def test_dp_special_cases():
    L = 7
    S = np.triu(np.ones((L, L)))
    a, v = oracle.dp_select_anchors(S, 1)
    assert a == [0] and abs(v - L) < 1e-15
    a, v = oracle.dp_select_anchors(S, L)
    assert a == list(range(L)) and abs(v - L) < 1e-15
    # uniform S: every choice is optimal; ties keep the smallest i
    a, v = oracle.dp_select_anchors(S, 3)
    assert abs(v - L) < 1e-15 and a[0] == 0


def test_dp_on_the_64k_end_to_end_similarity_matrix():
    # 36 layers, 6 anchors; the DP value equals the coverage of its own set
    S = synth.similarity_matrix(5, 36)
    a, v = oracle.dp_select_anchors(S, 6)
    assert len(a) == 6 and a[0] == 0
    assert abs(oracle.coverage_score(S, a) - v) < 1e-9

"""Pins for the oracle's offline anchor selection: eq. sim, eq. w and the DP."""
import itertools
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


# ---------------------------------------------------------------------------
# per-head similarity, head maps, remapped layer similarity
# ---------------------------------------------------------------------------

def test_sim_closed_form_small():
    # I_a = {0, 1}, I_b = {2, 3}: sim = (0.1 + 0.2) / (0.3 + 0.4) = 3/7
    pa = np.array([0.4, 0.3, 0.2, 0.1])
    pb = np.array([0.1, 0.2, 0.3, 0.4])
    assert abs(oracle.sim(pa, pb, 2) - 3.0 / 7.0) < 1e-15


def test_head_similarity_permuted_heads():
    """Layer b's heads are a permutation of layer a's: the per-head similarity
    is exactly 1 on the permutation, the head map recovers it, and the
    remapped layer similarity is 1."""
    rng = np.random.default_rng(3)
    S, H, N, k = 3, 4, 200, 20
    pa = rng.random((S, H, N)) ** 8
    perm = np.array([2, 0, 3, 1])
    pb = pa[:, perm, :]
    M = oracle.head_similarity(pa, pb, k)
    for gb in range(H):
        assert M[perm[gb], gb] == 1.0
        assert np.all(M[:, gb] <= 1.0 + 1e-15)
    assert np.array_equal(oracle.head_map_from_similarity(M), perm)
    assert oracle.remapped_layer_similarity(M) == 1.0


def test_head_similarity_matches_definition_by_brute_force():
    """Tiny rows: each Top-k set is the best k-subset by brute force."""
    rng = np.random.default_rng(4)
    S, H, N, k = 2, 2, 7, 3
    pa = rng.random((S, H, N))
    pb = rng.random((S, H, N))

    def best(p):
        return max(itertools.combinations(range(N), k), key=lambda c: (sum(p[list(c)]), [-x for x in c]))

    M = oracle.head_similarity(pa, pb, k)
    for ga in range(H):
        for gb in range(H):
            vals = []
            for s in range(S):
                Ia, Ib = list(best(pa[s, ga])), list(best(pb[s, gb]))
                vals.append(pb[s, gb, Ia].sum() / pb[s, gb, Ib].sum())
            assert abs(M[ga, gb] - np.mean(vals)) < 1e-14


def test_head_map_ties_go_to_lower_head():
    M = np.array([[0.5, 0.2], [0.5, 0.9], [0.1, 0.9]])
    assert list(oracle.head_map_from_similarity(M)) == [0, 1]
    assert abs(oracle.remapped_layer_similarity(M) - 0.7) < 1e-15

"""Pins for the oracle's Top-k selection and k rule (CPU only)."""
import itertools
import json
import os

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _brute_best_mass(s, k):
    """Largest total of any k-subset, by enumeration."""
    return max(sum(s[list(c)]) for c in itertools.combinations(range(len(s)), k))


def _rank_rule(s, k):
    """j is selected iff fewer than k positions beat it under (value desc, index asc)."""
    n = len(s)
    return [j for j in range(n)
            if sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j)) < k]


def test_topk_brute_force_tiny():
    r = np.random.default_rng(0)
    for n in range(1, 11):
        for _ in range(4):
            s = r.random(n)
            for k in range(0, n + 1):
                idx = oracle.topk_full_sort(s, k)
                assert len(idx) == k and list(idx) == sorted(set(idx.tolist()))
                if k:
                    assert abs(s[idx].sum() - _brute_best_mass(s, k)) < 1e-12
                assert idx.tolist() == _rank_rule(s, k)


def test_topk_matches_stable_argsort():
    r = np.random.default_rng(1)
    for n in (1, 2, 17, 257, 4099):
        s = np.round(r.standard_normal(n), 1)  # many ties
        for k in (1, 2, n // 3 + 1, n - 1, n):
            if k < 1:
                continue
            want = np.sort(np.argsort(-s, kind="stable")[:k])
            assert oracle.topk_full_sort(s, k).tolist() == want.tolist()


def test_topk_constant_row_and_k_ge_n():
    s = np.full(50, 0.25)
    assert oracle.topk_full_sort(s, 7).tolist() == list(range(7))
    assert oracle.topk_full_sort(s, 50).tolist() == list(range(50))
    assert oracle.topk_full_sort(s, 80).tolist() == list(range(50))


def test_topk_negative_zero_is_zero():
    s = np.array([-0.0, 0.0, -0.0, -1.0, 0.0])
    assert oracle.topk_full_sort(s, 2).tolist() == [0, 1]
    assert oracle.topk_full_sort(s, 4).tolist() == [0, 1, 2, 4]


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(min_value=-4, max_value=4), min_size=1, max_size=40),
       st.integers(min_value=1, max_value=40))
def test_topk_property_with_ties(vals, k):
    s = np.array(vals, dtype=np.float64) * 0.5
    k = min(k, len(s))
    idx = oracle.topk_full_sort(s, k)
    assert idx.tolist() == _rank_rule(s, k)


def test_k_rule_golden():
    g = json.load(open(os.path.join(GOLD, "k_rule.json")))
    for c in g["cases"]:
        assert oracle.topk_for_len(c["n"], k_min=g["decode_k_min"]) == c["k"], c
    for c in g["prefill_cases"]:
        assert oracle.prefill_tile_k(c["t"], 32768, tile=g["prefill_tile"],
                                     k_min=g["prefill_k_min"]) == (c["P_t"], c["k_t"]), c


def test_k_rule_is_nearest_multiple_of_64():
    for n in range(1280, 200000, 997):
        k = oracle.topk_for_len(n)
        assert k % 64 == 0
        assert abs(k - 0.1 * n) <= 32 + 1e-9


def test_index_set_acceptance_rule():
    s = np.array([5.0, 4.0, 3.0, 3.0 * (1 + 5e-6), 1.0])
    ref = oracle.topk_full_sort(s, 3)            # [0, 1, 3]
    assert oracle.index_sets_agree([0, 1, 2], ref, s)[0]  # 2 and 3 are within 1e-5
    assert not oracle.index_sets_agree([0, 1, 4], ref, s)[0]
    assert not oracle.index_sets_agree([0, 1], ref, s)[0]


def _brute_best_subset(s, k):
    """The k-subset of positions with the largest total, by enumeration (the
    maximiser is unique for rows of distinct values)."""
    best, best_set = -np.inf, None
    for c in itertools.combinations(range(len(s)), k):
        tot = s[list(c)].sum()
        if tot > best:
            best, best_set = tot, c
    return list(best_set)


def test_tile_topk_brute_force_per_tile_k_and_padding():
    """Tile Top-k ([Explainer] "Top-k設定", eq. k, with the query tiles of
    "実装のポイント"): each pooled row (b, t, g) of prefix length P_t keeps its
    best k_t-subset, ascending, then -1 up to k_max, the k of the LAST tile.

    Rule {tile 4, pct 50, round_to 2, k_min 3} over a 20-token prompt makes
    every tile's k different; by hand from eq. k:
      P_t = 4, 8, 12, 16, 20
      50% of P_t rounded to the nearest even number = 2, 4, 6, 8, 10
      at least 3, at most P_t -> k_t = 3, 4, 6, 8, 10 and k_max = 10."""
    n, tile = 20, 4
    want_P = [4, 8, 12, 16, 20]
    want_k = [3, 4, 6, 8, 10]
    r = np.random.default_rng(11)
    B, Hkv = 1, 2
    rows = [[[r.permutation(P).astype(np.float64) + r.random(P) * 0.5 for _ in range(Hkv)]
             for P in want_P] for _ in range(B)]
    idx = oracle.tile_topk(rows, n, tile=tile, pct=50, round_to=2, k_min=3)
    assert idx.shape == (B, len(want_P), Hkv, 10)
    for b in range(B):
        for t, (P, k_t) in enumerate(zip(want_P, want_k)):
            for g in range(Hkv):
                got = idx[b, t, g]
                assert got[:k_t].tolist() == _brute_best_subset(rows[b][t][g], k_t), (t, g)
                assert (got[k_t:] == -1).all(), (t, g)
                assert (got[:k_t] < P).all()


def test_tile_topk_k_max_comes_from_the_last_tile():
    """With a prompt that ends mid-tile, the last tile's prefix is the whole
    prompt: 10 tokens in tiles of 4 under {pct 50, round_to 2, k_min 1} give
    P_t = 4, 8, 10 and k_t = 2, 4, 6 (by hand), so rows are padded to 6."""
    r = np.random.default_rng(12)
    rows = [[[r.random(P) for _ in range(1)] for P in (4, 8, 10)]]
    idx = oracle.tile_topk(rows, 10, tile=4, pct=50, round_to=2, k_min=1)
    assert idx.shape == (1, 3, 1, 6)
    for t, k_t in enumerate((2, 4, 6)):
        assert idx[0, t, 0, :k_t].tolist() == _brute_best_subset(rows[0][t][0], k_t)
        assert (idx[0, t, 0, k_t:] == -1).all()

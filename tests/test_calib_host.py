"""Host-side calibration steps of the library (anchor DP, weighted
similarity, head maps) against the oracle on identical inputs.  No GPU: these
are plain host functions of libkascade.so."""
import numpy as np
import pytest

import oracle
from long_context_anchor_amd import kascade as K


def _lib_or_skip():
    try:
        K.lib()
    except (RuntimeError, OSError) as e:   # pragma: no cover
        pytest.skip("library not built: %s" % e)


@pytest.mark.parametrize("L,M,seed", [(1, 1, 0), (5, 2, 1), (10, 4, 2), (36, 6, 3), (36, 36, 4), (20, 1, 5)])
def test_select_anchors_matches_oracle_dp(L, M, seed):
    _lib_or_skip()
    rng = np.random.default_rng(seed)
    S = np.triu(rng.random((L, L)))
    np.fill_diagonal(S, 1.0)
    anchors, score = K.kascade_select_anchors(L, M, S)
    ra, rs = oracle.dp_select_anchors(S, M)
    assert anchors == ra
    assert abs(score - rs) <= 1e-12 * max(1.0, abs(rs))
    assert anchors[0] == 0


def test_select_anchors_rejects_bad_m():
    _lib_or_skip()
    S = np.eye(4)
    with pytest.raises(K.KascadeError):
        K.kascade_select_anchors(4, 5, S)
    with pytest.raises(K.KascadeError):
        K.kascade_select_anchors(4, 0, S)


def test_weighted_similarity_matches_oracle():
    _lib_or_skip()
    rng = np.random.default_rng(7)
    L, H = 6, 4
    sim = rng.random((L, L, H, H)).astype(np.float32)
    sim[2, 4, :, 1] = 0.5      # a tie across anchor heads
    w = rng.random(L).astype(np.float32)
    S = K.kascade_weighted_similarity(L, H, sim, w)
    for a in range(L):
        for b in range(L):
            if b < a:
                assert S[a, b] == 0.0
                continue
            want = float(w[b]) * oracle.remapped_layer_similarity(sim[a, b])
            assert abs(S[a, b] - want) <= 1e-12
    S1 = K.kascade_weighted_similarity(L, H, sim, None)
    assert abs(S1[1, 3] - oracle.remapped_layer_similarity(sim[1, 3])) <= 1e-12


def test_head_maps_match_oracle():
    _lib_or_skip()
    rng = np.random.default_rng(8)
    L, H = 9, 8
    sim = rng.random((L, L, H, H)).astype(np.float32)
    sim[0, 1, 3, 2] = sim[0, 1, 5, 2] = 2.0   # tie: the lower anchor head wins
    anchors = [0, 4, 7]
    hm = K.kascade_head_maps(L, H, sim, anchors)
    for b in range(L):
        a = oracle.anchor_of(b, anchors)
        if a == b:
            assert list(hm[b]) == list(range(H))
        else:
            assert list(hm[b]) == list(oracle.head_map_from_similarity(sim[a, b]))
    assert hm[1, 2] == 3
    with pytest.raises(K.KascadeError):
        K.kascade_head_maps(L, H, sim, [1, 4])

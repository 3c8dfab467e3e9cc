"""Pins for the oracle's attention functions (CPU only).

Each check ties the oracle to something other than itself: torch's
scaled_dot_product_attention (a library routine) in float64, closed forms from
tests/golden/, and invariants of softmax attention.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, G, causal=False, mask=None):
    """Library routine: torch SDPA in float64 on CPU, KV heads expanded h -> h//G."""
    q, k, v = (np.array(x, dtype=np.float64) for x in (q, k, v))
    tq = torch.as_tensor(q, dtype=torch.float64)
    tk = torch.as_tensor(k, dtype=torch.float64).repeat_interleave(G, dim=1)
    tv = torch.as_tensor(v, dtype=torch.float64).repeat_interleave(G, dim=1)
    m = None if mask is None else torch.as_tensor(mask)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m,
                                                            is_causal=causal).numpy()


def test_dense_decode_matches_library_sdpa():
    B, Hq, Hkv, d, N = 2, 4, 2, 16, 37
    q, k, v = _rand((B, Hq, d), 1), _rand((B, Hkv, N, d), 2), _rand((B, Hkv, N, d), 3)
    out, lse, p = oracle.dense_decode(q, k, v)
    ref = _sdpa(q[:, :, None, :], k, v, Hq // Hkv)[:, :, 0, :]
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.allclose(p.sum(-1), 1.0, atol=1e-13)


def test_dense_decode_probabilities_match_library_with_identity_values():
    # SDPA with V = identity returns the attention matrix itself.
    B, Hq, Hkv, d, N = 1, 4, 2, 8, 19
    q, k = _rand((B, Hq, d), 4), _rand((B, Hkv, N, d), 5)
    eye = np.broadcast_to(np.eye(N), (B, Hkv, N, N))
    _, _, p = oracle.dense_decode(q, k, eye)
    ref = _sdpa(q[:, :, None, :], k, eye, Hq // Hkv)[:, :, 0, :]
    assert np.max(np.abs(p - ref)) < 1e-13


def test_decode_closed_form_golden():
    g = json.load(open(os.path.join(GOLD, "decode_closed_form.json")))
    q = np.array(g["q"])[None, None, :]
    k = np.zeros((1, 1, 4, 4))
    k[0, 0, :, 0] = [math.log(j + 1) for j in range(4)]
    v = np.array(g["v"], dtype=np.float64)[None, None]
    out, lse, p = oracle.dense_decode(q, k, v)
    assert np.allclose(p[0, 0], g["p"], atol=1e-15)
    assert abs(lse[0, 0] - math.log(10.0)) < 1e-14
    assert np.allclose(out[0, 0], g["out"], atol=1e-14)
    pooled = oracle.pool_decode(p, 1)
    idx = oracle.topk_full_sort(pooled[0, 0], 2)
    assert idx.tolist() == g["top2"]
    sp, _ = oracle.sparse_decode(q, k, v, idx[None, None, :])
    assert np.allclose(sp[0, 0], g["sparse_top2_out"], atol=1e-14)


def test_dense_decode_special_cases():
    q, k, v = _rand((1, 2, 8), 6), _rand((1, 1, 1, 8), 7), _rand((1, 1, 1, 8), 8)
    out, _, _ = oracle.dense_decode(q, k, v)
    assert np.allclose(out[0, 0], v[0, 0, 0]) and np.allclose(out[0, 1], v[0, 0, 0])
    # equal scores (q = 0) give the mean of V
    v2 = _rand((1, 1, 9, 8), 9)
    out, _, p = oracle.dense_decode(np.zeros((1, 1, 8)), _rand((1, 1, 9, 8), 10), v2)
    assert np.allclose(out[0, 0], v2[0, 0].mean(0), atol=1e-15)
    assert np.allclose(p, 1.0 / 9)


def test_pool_decode_mass_and_group_one():
    B, Hq, Hkv, d, N = 2, 8, 2, 8, 50
    q, k, v = _rand((B, Hq, d), 11), _rand((B, Hkv, N, d), 12), _rand((B, Hkv, N, d), 13)
    _, _, p = oracle.dense_decode(q, k, v)
    pooled = oracle.pool_decode(p, Hkv)
    assert np.allclose(pooled.sum(-1), Hq // Hkv, atol=1e-12)
    # group 0 collects exactly heads 0..3 (a wrong head->KV mapping fails this)
    assert np.allclose(pooled[:, 0], p[:, 0:4].sum(1))
    # G = 1: Top-k of P is the argsort of the raw logits (softmax is monotone)
    q1 = _rand((1, 1, d), 14)
    k1 = _rand((1, 1, N, d), 15)
    _, _, p1 = oracle.dense_decode(q1, k1, k1)
    logits = k1[0, 0] @ q1[0, 0]
    for kk in (1, 5, 17, N):
        want = np.sort(np.argsort(-logits, kind="stable")[:kk])
        assert oracle.topk_full_sort(oracle.pool_decode(p1, 1)[0, 0], kk).tolist() == want.tolist()


def test_sparse_decode_matches_masked_library_sdpa():
    B, Hq, Hkv, d, N, K = 2, 4, 2, 8, 40, 11
    q, k, v = _rand((B, Hq, d), 16), _rand((B, Hkv, N, d), 17), _rand((B, Hkv, N, d), 18)
    r = np.random.default_rng(19)
    idx = np.stack([np.stack([np.sort(r.choice(N, K, replace=False)) for _ in range(Hkv)])
                    for _ in range(B)])
    head_map = [1, 0]
    out, _ = oracle.sparse_decode(q, k, v, idx, head_map)
    mask = np.zeros((B, Hq, 1, N), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            mask[b, h, 0, idx[b, head_map[h // 2]]] = True
    ref = _sdpa(q[:, :, None, :], k, v, 2, mask=mask)[:, :, 0, :]
    assert np.max(np.abs(out - ref)) < 1e-12


def test_sparse_decode_full_set_equals_dense_and_k1_picks_row():
    B, Hq, Hkv, d, N = 1, 4, 2, 16, 33
    q, k, v = _rand((B, Hq, d), 20), _rand((B, Hkv, N, d), 21), _rand((B, Hkv, N, d), 22)
    dense, _, _ = oracle.dense_decode(q, k, v)
    full = np.broadcast_to(np.arange(N), (B, Hkv, N))
    sp, _ = oracle.sparse_decode(q, k, v, full)
    assert np.max(np.abs(sp - dense)) < 1e-12
    # permuting the list changes nothing
    perm = np.random.default_rng(23).permutation(N)
    sp2, _ = oracle.sparse_decode(q, k, v, full[..., perm])
    assert np.max(np.abs(sp2 - dense)) < 1e-12
    one = np.full((B, Hkv, 1), 7)
    sp1, _ = oracle.sparse_decode(q, k, v, one)
    assert np.allclose(sp1[0, 0], v[0, 0, 7]) and np.allclose(sp1[0, 3], v[0, 1, 7])


def test_dense_prefill_matches_causal_library_sdpa():
    B, Hq, Hkv, d, N = 1, 4, 2, 16, 45
    q, k, v = _rand((B, Hq, N, d), 24), _rand((B, Hkv, N, d), 25), _rand((B, Hkv, N, d), 26)
    out, lse = oracle.dense_prefill(q, k, v)
    ref = _sdpa(q, k, v, 2, causal=True)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_tile_pool_matches_library_probabilities():
    # P from SDPA with V = identity and a causal mask; pooled = sums over the
    # tile's rows and the group's heads.
    B, Hq, Hkv, d, N, tile = 1, 4, 2, 8, 21, 8
    q, k = _rand((B, Hq, N, d), 27), _rand((B, Hkv, N, d), 28)
    eye = np.broadcast_to(np.eye(N), (B, Hkv, N, N))
    P = _sdpa(q, k, eye, 2, causal=True)  # [B,Hq,N,N]
    rows = oracle.tile_pool(q, k, tile)
    T = -(-N // tile)
    for t in range(T):
        lo, hi = tile * t, min(N, tile * (t + 1))
        for g in range(Hkv):
            want = P[0, 2 * g:2 * g + 2, lo:hi, :hi].sum(axis=(0, 1))
            got = rows[0][t][g]
            assert got.shape == (hi,)
            assert np.max(np.abs(got - want)) < 1e-12
            # mass: every row sums to one
            assert abs(got.sum() - 2 * (hi - lo)) < 1e-11


def test_tile_pool_tile_one_is_per_row_probability():
    B, Hq, Hkv, d, N = 1, 1, 1, 8, 9
    q, k, v = _rand((B, Hq, N, d), 29), _rand((B, Hkv, N, d), 30), _rand((B, Hkv, N, d), 31)
    rows = oracle.tile_pool(q, k, tile=1)
    for r in range(N):
        _, _, p = oracle.dense_prefill_rows(q, k, v, 0, 0, [r])
        assert np.allclose(rows[0][r][0], p[0, : r + 1], atol=1e-15)


def test_sparse_prefill_matches_masked_library_sdpa():
    B, Hq, Hkv, d, N, tile = 1, 4, 2, 8, 37, 8
    q, k, v = _rand((B, Hq, N, d), 32), _rand((B, Hkv, N, d), 33), _rand((B, Hkv, N, d), 34)
    T = -(-N // tile)
    r = np.random.default_rng(35)
    kmax = 12
    idx = -np.ones((B, T, Hkv, kmax), dtype=np.int64)
    for t in range(T):
        P_t = min(N, tile * (t + 1))
        kt = min(P_t, kmax)
        for g in range(Hkv):
            sel = np.sort(r.choice(P_t, kt, replace=False))
            # guarantee every row sees at least one key: include key 0
            if 0 not in sel:
                sel[0] = 0
                sel = np.sort(sel)
            idx[0, t, g, :kt] = sel
    head_map = [1, 0]
    out = oracle.sparse_prefill(q, k, v, idx, head_map, tile)
    mask = np.zeros((B, Hq, N, N), dtype=bool)
    for h in range(Hq):
        for rr in range(N):
            J = idx[0, rr // tile, head_map[h // 2]]
            J = J[(J >= 0) & (J <= rr)]
            mask[0, h, rr, J] = True
    ref = _sdpa(q, k, v, 2, mask=mask)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_sparse_prefill_full_lists_equal_dense():
    B, Hq, Hkv, d, N, tile = 1, 2, 1, 8, 20, 8
    q, k, v = _rand((B, Hq, N, d), 36), _rand((B, Hkv, N, d), 37), _rand((B, Hkv, N, d), 38)
    T = -(-N // tile)
    idx = -np.ones((B, T, Hkv, N), dtype=np.int64)
    for t in range(T):
        P_t = min(N, tile * (t + 1))
        idx[0, t, 0, :P_t] = np.arange(P_t)
    dense, _ = oracle.dense_prefill(q, k, v)
    sp = oracle.sparse_prefill(q, k, v, idx, [0], tile)
    assert np.max(np.abs(sp - dense)) < 1e-12


def test_anchor_and_reuse_decode_layers_against_library_routines():
    """One anchor decode layer and the reuse layer that reads its lists
    ([Explainer] "アンカーレイヤーと再利用レイヤー", "ヘッドリマッピング"): the
    anchor's output equals torch SDPA over all keys and its lse the log of the
    row sums; its pooled row per KV head is SDPA's probabilities summed over
    the group's heads; its list is the topk best keys of that row by a stable
    library sort, ascending; the reuse layer equals SDPA under the boolean
    mask of the remapped lists."""
    B, Hq, Hkv, d, N, topk = 2, 6, 3, 8, 40, 7
    G = Hq // Hkv
    q, k, v = _rand((B, Hq, 1, d), 66), _rand((B, Hkv, N, d), 67), _rand((B, Hkv, N, d), 68)
    out, lse, pooled, idx = oracle.anchor_decode(q[:, :, 0], k, v, topk)
    assert np.max(np.abs(out - _sdpa(q, k, v, G)[:, :, 0])) < 1e-12
    s = np.einsum("bhd,bhmd->bhm", q[:, :, 0], np.repeat(k, G, axis=1)) / math.sqrt(d)
    assert np.max(np.abs(lse - np.log(np.exp(s).sum(-1)))) < 1e-12
    P = _sdpa(q, k, np.broadcast_to(np.eye(N), (B, Hkv, N, N)), G)[:, :, 0]
    assert idx.shape == (B, Hkv, topk)
    for b in range(B):
        for g in range(Hkv):
            assert np.max(np.abs(pooled[b, g] - P[b, G * g:G * g + G].sum(axis=0))) < 1e-12
            best = np.argsort(-pooled[b, g], kind="stable")[:topk]
            assert idx[b, g].tolist() == sorted(best.tolist()), (b, g)
    q2, k2, v2 = _rand((B, Hq, 1, d), 69), _rand((B, Hkv, N, d), 70), _rand((B, Hkv, N, d), 71)
    head_map = [2, 0, 0]
    got = oracle.reuse_decode(q2[:, :, 0], k2, v2, idx, head_map)
    mask = np.zeros((B, Hq, 1, N), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            mask[b, h, 0, idx[b, head_map[h // G]]] = True
    assert np.max(np.abs(got - _sdpa(q2, k2, v2, G, mask=mask)[:, :, 0])) < 1e-12


def test_anchor_and_reuse_prefill_layers_against_library_routines():
    """One anchor prefill layer and the reuse layer that reads its lists
    ([Explainer] "アンカーレイヤーと再利用レイヤー", "ヘッドリマッピング", "Top-k設定"
    eq. k with the query tiles of "実装のポイント"): the anchor's output equals
    causal torch SDPA and its lse the log of the causal row sums; its pooled
    rows equal SDPA's probabilities summed over each tile's rows and the
    group's heads; its lists are the k_t best keys of each pooled row by a
    stable library sort (ties to the lower index), ascending, then -1 up to
    k_max; the reuse layer equals SDPA under the boolean mask those lists and
    the head map define.  Rule {tile 4, pct 50, round_to 2, k_min 4} on a
    20-token prompt gives, by hand, P_t = 4, 8, 12, 16, 20 and k_t = 4, 4, 6,
    8, 10 (k_min >= tile, so no reuse row is left without keys)."""
    B, Hq, Hkv, d, N, tile = 1, 4, 2, 8, 20, 4
    G = Hq // Hkv
    want_k = [4, 4, 6, 8, 10]
    q, k, v = _rand((B, Hq, N, d), 60), _rand((B, Hkv, N, d), 61), _rand((B, Hkv, N, d), 62)
    out, lse, pooled, idx = oracle.anchor_prefill(q, k, v, tile=tile, pct=50, round_to=2, k_min=4)
    assert np.max(np.abs(out - _sdpa(q, k, v, G, causal=True))) < 1e-12
    s = np.einsum("bhnd,bhmd->bhnm", q, np.repeat(k, G, axis=1)) / math.sqrt(d)
    s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    assert np.max(np.abs(lse - np.log(np.exp(s).sum(-1)))) < 1e-12
    P = _sdpa(q, k, np.broadcast_to(np.eye(N), (B, Hkv, N, N)), G, causal=True)
    assert idx.shape == (B, len(want_k), Hkv, want_k[-1])
    for t, k_t in enumerate(want_k):
        lo, hi = tile * t, tile * (t + 1)
        for g in range(Hkv):
            row = np.asarray(pooled[0][t][g])
            assert np.max(np.abs(row - P[0, G * g:G * g + G, lo:hi, :hi].sum(axis=(0, 1)))) < 1e-12
            best = np.argsort(-row, kind="stable")[:k_t]
            assert idx[0, t, g, :k_t].tolist() == sorted(best.tolist()), (t, g)
            assert (idx[0, t, g, k_t:] == -1).all(), (t, g)
    q2, k2, v2 = _rand((B, Hq, N, d), 63), _rand((B, Hkv, N, d), 64), _rand((B, Hkv, N, d), 65)
    head_map = [1, 0]
    got = oracle.reuse_prefill(q2, k2, v2, idx, head_map, tile=tile)
    mask = np.zeros((B, Hq, N, N), dtype=bool)
    for h in range(Hq):
        for r in range(N):
            J = idx[0, r // tile, head_map[h // G]]
            mask[0, h, r, J[(J >= 0) & (J <= r)]] = True
    assert mask.any(axis=-1).all()
    assert np.max(np.abs(got - _sdpa(q2, k2, v2, G, mask=mask))) < 1e-12


def test_anchor_prefill_tiles_zero_and_one_are_dense():
    # with the prefill k rule (minimum 256, tile 128) tiles 0 and 1 keep every key
    for t, P in ((0, 128), (1, 256)):
        assert oracle.prefill_tile_k(t, 32768) == (P, P)


def test_oracle_rejects_non_finite():
    q = np.zeros((1, 1, 4))
    k = np.zeros((1, 1, 3, 4))
    k[0, 0, 1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.dense_decode(q, k, k)
    with pytest.raises(ValueError):
        oracle.topk_full_sort(np.array([1.0, np.inf]), 1)


def _planted_stack(seed=21):
    """A 5-layer decode stack, anchors [0, 3], 2 KV heads of 2 query heads,
    whose anchors each put nearly all attention on one known key per KV head.

    Every query is e_0 and anchor layer a's KV head c has key 40 e_0 at
    position pos[a][c] (the other keys are below 0.05 in every entry), so the
    pooled row's unique maximum is pos[a][c]."""
    r = np.random.default_rng(seed)
    L, B, Hq, Hkv, d, N = 5, 1, 4, 2, 8, 16
    anchors = [0, 3]
    pos = {0: [5, 11], 3: [2, 14]}
    maps = {1: [1, 0], 2: [0, 0], 4: [1, 1]}
    layers = []
    for l in range(L):
        q = np.zeros((B, Hq, d))
        q[..., 0] = 1.0
        k = r.uniform(-0.05, 0.05, (B, Hkv, N, d))
        v = r.standard_normal((B, Hkv, N, d))
        if l in anchors:
            for c in range(Hkv):
                k[0, c, pos[l][c]] = 0.0
                k[0, c, pos[l][c], 0] = 40.0
        layers.append({"q": q, "k": k, "v": v})
    return layers, anchors, maps, pos


def test_layer_stack_with_one_selected_key_is_closed_form():
    """Layer stack ([Explainer] "アンカーレイヤーと再利用レイヤー": a reuse layer
    attends only to the keys its nearest preceding anchor selected;
    "ヘッドリマッピング": reuse KV head g takes anchor KV head head_map[g]'s list
    and its own K/V).  With k = 1 a reuse layer's output for query head h is
    exactly the row of ITS OWN V at the one selected position:
      layer 1 (anchor 0, map [1,0]): head g -> v_1[g][pos[0][1-g]]
      layer 2 (anchor 0, map [0,0]): both heads -> v_2[g][pos[0][0]]
      layer 4 (anchor 3, map [1,1]): both heads -> v_4[g][pos[3][1]]."""
    layers, anchors, maps, pos = _planted_stack()
    outs, idx = oracle.run_decode_layerstack(layers, anchors, maps, topk=1)
    assert sorted(idx) == anchors
    for a in anchors:
        assert idx[a][0, :, 0].tolist() == pos[a]
    want_pos = {1: [pos[0][1], pos[0][0]], 2: [pos[0][0], pos[0][0]], 4: [pos[3][1], pos[3][1]]}
    for l, wp in want_pos.items():
        v = layers[l]["v"]
        for h in range(4):
            g = h // 2
            assert np.max(np.abs(outs[l][0, h] - v[0, g, wp[g]])) == 0.0, (l, h)
    # anchors are exact dense attention (torch SDPA in fp64)
    for a in anchors:
        lay = layers[a]
        ref = _sdpa(lay["q"][:, :, None, :], lay["k"], lay["v"], 2)[:, :, 0, :]
        assert np.max(np.abs(outs[a] - ref)) < 1e-12


def test_layer_stack_with_full_lists_is_dense_everywhere():
    """k = N: every reuse layer's list is the whole cache, so every layer of
    the stack equals dense attention of its own q, k, v (torch SDPA)."""
    layers, anchors, maps, _ = _planted_stack(seed=22)
    for lay in layers:
        lay["q"] = _rand(lay["q"].shape, 23)
    outs, _ = oracle.run_decode_layerstack(layers, anchors, maps, topk=16)
    for l, lay in enumerate(layers):
        ref = _sdpa(lay["q"][:, :, None, :], lay["k"], lay["v"], 2)[:, :, 0, :]
        assert np.max(np.abs(outs[l] - ref)) < 1e-12, l

"""GPU parity of the prefill path (anchor flash + tile pooling + tile Top-k,
reuse gathered attention) against the fp64 oracle, through the C ABI.

Tolerances (bf16 inputs): outputs max-abs 2e-2; lse 1e-3 (fp32 statistics of
bf16 products); pooled rows 1e-3 relative (P is formed in fp32 from the same
bf16 products); indices bit-exact against a full sort of the GPU's own pooled
row, and within the 1e-5 relative band against the oracle's pooled row.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_anchor_amd import configs, synth
from long_context_anchor_amd import kascade as K

pytestmark = pytest.mark.gpu

DEV = "cuda"
RULE = K.PREFILL_RULE


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _rand_layer(B, Hq, Hkv, N, seed, planted=False):
    if planted:
        cfg = configs.LLAMA_PREFILL_32K
        lin = synth.heavy_lineages(seed, 1, Hkv, N, max(1, N // 10), cfg.drift)
        return synth.prefill_layer(seed, 0, B, Hq, Hkv, 128, N, lin[0], cfg.alpha, cfg.gamma,
                                   "bf16", device=DEV)
    g = torch.Generator(device=DEV).manual_seed(seed)
    q = torch.randn((B, Hq, N, 128), generator=g, device=DEV).bfloat16()
    k = torch.randn((B, Hkv, N, 128), generator=g, device=DEV).bfloat16()
    v = torch.randn((B, Hkv, N, 128), generator=g, device=DEV).bfloat16()
    return q, k, v


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 1, 1, 1), (1, 2, 1, 128), (2, 4, 2, 200),
                                        (1, 8, 2, 384), (1, 8, 1, 1000), (1, 16, 2, 257)])
def test_dense_prefill_parity(B, Hq, Hkv, N):
    say("dense prefill", B, Hq, Hkv, N)
    q, k, v = _rand_layer(B, Hq, Hkv, N, seed=N + Hq)
    out, lse = K.dense_prefill(q, k, v)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_prefill(np64(q), np64(k), np64(v))
    assert np.max(np.abs(np64(out) - ro)) <= 2e-2
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-3


def _check_anchor_prefill(q, k, v, tiles=None, heads_g=None):
    """Run the anchor prefill and compare sampled (t, g) rows with the oracle.
    Returns the GPU idx and the oracle idx rows computed."""
    B, Hq, N, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    T = -(-N // 128)
    out, lse, idx, pooled = K.anchor_prefill(q, k, v, RULE, want_pooled=True)
    torch.cuda.synchronize()
    qn, kn, vn = np64(q), np64(k), np64(v)
    gidx = idx.cpu().numpy()
    gpool = pooled.cpu().numpy()
    tiles = range(T) if tiles is None else tiles
    heads_g = range(Hkv) if heads_g is None else heads_g
    ref_idx = {}
    for b in range(B):
        for t in tiles:
            P, kt = oracle.prefill_tile_k(t, N)
            rows = range(128 * t, min(N, 128 * (t + 1)))
            for g in heads_g:
                for h in (g * G, g * G + G - 1):
                    ro, rl, _ = oracle.dense_prefill_rows(qn, kn, vn, b, h, rows)
                    assert np.max(np.abs(np64(out[b, h, 128 * t:128 * t + len(rows)]) - ro)) <= 2e-2
                    assert np.max(np.abs(np64(lse[b, h, 128 * t:128 * t + len(rows)]) - rl)) <= 1e-3
                rp = oracle.tile_pool_one(qn, kn, b, t, g)
                gp = K.packed_row(torch.as_tensor(gpool[b]), t, g, N, Hkv).numpy().astype(np.float64)
                assert gp.shape == rp.shape
                assert np.max(np.abs(gp - rp) / np.maximum(rp, 1e-6)) <= 1e-3
                row = gidx[b, t, g]
                assert np.all(row[kt:] == -1)
                sel = row[:kt]
                assert np.all(np.diff(sel) > 0)
                assert np.array_equal(sel, oracle.topk_full_sort(gp, kt))
                ri = oracle.topk_full_sort(rp, kt)
                ok, nd = oracle.index_sets_agree(sel, ri, rp)
                assert ok, (b, t, g, nd)
                ref_idx[(b, t, g)] = ri
    return out, idx, ref_idx


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 4, 1, 1), (2, 4, 2, 37), (1, 4, 1, 128), (1, 8, 2, 300),
                                        (2, 4, 2, 640), (1, 4, 4, 1000), (1, 16, 2, 2049)])
def test_anchor_prefill_parity(B, Hq, Hkv, N):
    say("anchor prefill", B, Hq, Hkv, N)
    q, k, v = _rand_layer(B, Hq, Hkv, N, seed=7 * N + Hq, planted=True)
    _check_anchor_prefill(q, k, v)


@pytest.mark.parametrize("Hq,Hkv,N,hm", [(4, 2, 1, [1, 1]), (4, 2, 37, [1, 0]), (4, 1, 300, [0]),
                                         (8, 2, 1000, [1, 0]),
                                         (8, 4, 2049, [2, 2, 0, 1]), (16, 2, 3000, [1, 1])])
def test_reuse_prefill_parity(Hq, Hkv, N, hm):
    say("reuse prefill", Hq, Hkv, N, hm)
    # anchor lists from the oracle's own pooled selection on an anchor layer
    qa, ka, va = _rand_layer(1, Hq, Hkv, N, seed=N, planted=True)
    qn, kn = np64(qa), np64(ka)
    T = -(-N // 128)
    kmax = oracle.prefill_tile_k(T - 1, N)[1]
    lists = -np.ones((1, T, Hkv, kmax), dtype=np.int32)
    for t in range(T):
        _, kt = oracle.prefill_tile_k(t, N)
        for g in range(Hkv):
            lists[0, t, g, :kt] = oracle.topk_full_sort(oracle.tile_pool_one(qn, kn, 0, t, g), kt)
    q, k, v = _rand_layer(1, Hq, Hkv, N, seed=N + 1, planted=True)
    out = K.reuse_prefill(q, k, v, torch.as_tensor(lists, device=DEV), hm, RULE)
    torch.cuda.synchronize()
    ref = oracle.sparse_prefill(np64(q), np64(k), np64(v), lists, hm)
    assert np.max(np.abs(np64(out) - ref)) <= 2e-2


def test_reuse_prefill_full_lists_equal_dense():
    N, Hq, Hkv = 700, 4, 2
    q, k, v = _rand_layer(1, Hq, Hkv, N, seed=11)
    T = -(-N // 128)
    # a rule whose k_t is the whole prefix: pct 100
    rule = K.TopkRule(128, 100, 64, 256)
    kmax = K.kascade_topk_for_len(N, rule)
    lists = -np.ones((1, T, Hkv, kmax), dtype=np.int32)
    for t in range(T):
        P = min(N, 128 * (t + 1))
        assert K.kascade_topk_for_len(P, rule) == P
        lists[0, t, :, :P] = np.arange(P)
    sp = K.reuse_prefill(q, k, v, torch.as_tensor(lists, device=DEV), [0, 1], rule)
    dense, _ = K.dense_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(sp.float() - dense.float())).item() <= 1e-2


def test_reuse_prefill_longest_list():
    """The longest list the contiguous reuse prefill stages in LDS (24576
    keys, checked on the host): with k_t the whole prefix (pct 100) the
    reuse pass is dense causal attention ([Explainer] "アンカーレイヤーと
    再利用レイヤー": softmax over the listed keys), here against the oracle's
    fp64 rows and the GPU's own dense pass."""
    N, Hq, Hkv = 24576, 2, 1
    say("reuse prefill longest list", N)
    q, k, v = _rand_layer(1, Hq, Hkv, N, seed=29)
    rule = K.TopkRule(128, 100, 64, 256)
    kmax = K.kascade_topk_for_len(N, rule)
    assert kmax == 24576
    T = N // 128
    lists = -np.ones((1, T, Hkv, kmax), dtype=np.int32)
    for t in range(T):
        lists[0, t, 0, :128 * (t + 1)] = np.arange(128 * (t + 1))
    sp = K.reuse_prefill(q, k, v, torch.as_tensor(lists, device=DEV), [0], rule)
    dense, _ = K.dense_prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(sp.float() - dense.float())).item() <= 1e-2
    qn, kn, vn, sn = np64(q), np64(k), np64(v), np64(sp)
    rows = [0, 1, 127, 128, 12345, N - 129, N - 1]
    for h in range(Hq):
        ro, _, _ = oracle.dense_prefill_rows(qn, kn, vn, 0, h, rows)
        assert np.max(np.abs(sn[0, h, rows] - ro)) <= 2e-2, h


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_llama_prefill_32k_sampled(dtype):
    """Full-size anchor + reuse layer pair of the 32K-token prefill workload
    (bf16, and the same workload in fp16); the oracle checks sampled tiles
    (0, 1, 20, 131, 255) of KV heads 0 and 6."""
    cfg = configs.LLAMA_PREFILL_32K
    N = cfg.ctx_len
    say("32K prefill anchor + reuse, sampled tiles", dtype)
    lin = synth.heavy_lineages(cfg.seed, 2, cfg.n_kv_heads, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, 2, cfg.anchors, cfg.n_kv_heads, cfg.head_map_kind)
    qa, ka, va = synth.prefill_layer(cfg.seed, 0, 1, cfg.n_q_heads, cfg.n_kv_heads, 128, N,
                                     synth.layer_heavy_sets(lin, 0, cfg.anchors, maps),
                                     cfg.alpha, cfg.gamma, dtype, device=DEV)
    tiles = [0, 1, 20, 131, 255]
    _, idx, ref_idx = _check_anchor_prefill(qa, ka, va, tiles=tiles, heads_g=[0, 6])
    hm = maps[1]
    q, k, v = synth.prefill_layer(cfg.seed, 1, 1, cfg.n_q_heads, cfg.n_kv_heads, 128, N,
                                  synth.layer_heavy_sets(lin, 1, cfg.anchors, maps),
                                  cfg.alpha, cfg.gamma, dtype, device=DEV)
    out = K.reuse_prefill(q, k, v, idx, hm, RULE)
    torch.cuda.synchronize()
    qn, kn, vn = np64(q), np64(k), np64(v)
    G = cfg.group
    # the oracle's own anchor lists for the sampled tiles (no GPU value feeds the oracle)
    T = N // 128
    olists = -np.ones((1, T, cfg.n_kv_heads, idx.shape[-1]), dtype=np.int64)
    for (b, t, g), ri in ref_idx.items():
        olists[b, t, g, :len(ri)] = ri
    for t in tiles:
        for g2 in range(cfg.n_kv_heads):
            if int(hm[g2]) not in (0, 6):
                continue
            rows = list(range(128 * t, 128 * t + 128, 9))
            h = g2 * G + 1
            ref = oracle.sparse_prefill_rows(qn, kn, vn, olists, hm, 0, h, rows)
            got = np64(out[0, h, rows])
            assert np.max(np.abs(got - ref)) <= 2e-2


def test_prefill_deterministic():
    q, k, v = _rand_layer(1, 8, 2, 1500, seed=3, planted=True)
    o1, l1, i1, p1 = K.anchor_prefill(q, k, v, RULE, want_pooled=True)
    o2, l2, i2, p2 = K.anchor_prefill(q, k, v, RULE, want_pooled=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2) and torch.equal(i1, i2) and torch.equal(p1, p2)


def test_prefill_sharp_softmax_and_late_max():
    """Sharp distributions and late maxima: every query has a component of 30
    along one unit direction w (plus 3 x N(0,1) noise), and the last key of
    every tile is 12 w, so those keys score about 30 above the rest and each
    row's reference max jumps when its key sequence reaches key 127."""
    say("prefill sharp softmax, late max")
    B, Hq, Hkv, N = 1, 8, 2, 700
    g = torch.Generator(device=DEV).manual_seed(98)
    w = torch.randn((128,), generator=g, device=DEV)
    w = w / w.norm()
    q = 3.0 * torch.randn((B, Hq, N, 128), generator=g, device=DEV) + 30.0 * w
    k = torch.randn((B, Hkv, N, 128), generator=g, device=DEV)
    v = torch.randn((B, Hkv, N, 128), generator=g, device=DEV).bfloat16()
    k[:, :, 127::128] = 12.0 * w
    q, k = q.bfloat16(), k.bfloat16()
    _check_anchor_prefill(q, k, v)


def test_prefill_graph_replay():
    """An anchor prefill and the reuse prefill that consumes its tile lists,
    captured as one HIP graph (workspace and outputs preallocated): each of
    three replays, with the outputs poisoned and eager work in between,
    equals the eager run bit for bit."""
    N, Hq, Hkv = 1000, 8, 2
    say("prefill graph replay", N, Hq, Hkv)
    qa, ka, va = _rand_layer(1, Hq, Hkv, N, seed=21, planted=True)
    qr, kr, vr = _rand_layer(1, Hq, Hkv, N, seed=22, planted=True)
    sh = K.make_shape(qa, ka, N)
    T, kmax = -(-N // 128), K.prefill_k_max(N, RULE)
    ws = K.workspace(K.OP_ANCHOR_PREFILL, sh, 0, RULE)
    out_a = torch.empty_like(qa)
    lse = torch.empty(qa.shape[:3], dtype=torch.float32, device=DEV)
    idx = torch.empty((1, T, Hkv, kmax), dtype=torch.int32, device=DEV)
    out_r = torch.empty_like(qr)

    def layer_pair():
        K.check(K.kascade_anchor_prefill(sh, qa, ka, va, RULE, out_a, lse, idx, None, ws, ws.numel()), "anchor")
        K.check(K.kascade_reuse_prefill(sh, qr, kr, vr, RULE, idx, [1, 0], out_r, None, 0), "reuse")

    layer_pair()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out_a, lse, idx, out_r)]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            layer_pair()
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(3):
        out_a.zero_()
        lse.fill_(float("nan"))
        idx.fill_(-7)
        out_r.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out_a, lse, idx, out_r), eager):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), rep
        layer_pair()   # eager work between replays
        torch.cuda.synchronize()

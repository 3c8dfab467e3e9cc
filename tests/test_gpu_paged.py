"""GPU parity of decode and of the gathered reuse prefill over paged KV caches
(block tables, layout [num_blocks, Hkv, block_size, d], blocks scattered by a
seeded permutation, ragged last block) against the oracle on the logical
caches.  Tolerances as for the contiguous calls: outputs 2e-2 max-abs (bf16),
lse 1e-4, pooled 1e-4 relative, indices bit-exact against a full sort of the
GPU's own pooled row and within the 1e-5 tie band of the oracle's.  The paged
reuse prefill reads the same rows with the same arithmetic as the contiguous
one, so the two must agree bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_anchor_amd import configs, synth
from long_context_anchor_amd import kascade as K

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _paged(k, v, bs, seed, spare=3):
    """Scatter contiguous caches [B, Hkv, N, d] into blocks; returns
    (k_cache, v_cache, block_table)."""
    B, Hkv, N, d = k.shape
    nb = -(-N // bs)
    total = B * nb + spare
    rng = np.random.default_rng(seed)
    perm = rng.permutation(total)[: B * nb].reshape(B, nb)
    kc = torch.zeros((total, Hkv, bs, d), dtype=k.dtype, device=DEV)
    vc = torch.zeros_like(kc)
    for b in range(B):
        for i in range(nb):
            lo, hi = i * bs, min(N, (i + 1) * bs)
            kc[perm[b, i], :, : hi - lo] = k[b, :, lo:hi]
            vc[perm[b, i], :, : hi - lo] = v[b, :, lo:hi]
    table = torch.full((B, nb + 2), -1, dtype=torch.int32, device=DEV)
    table[:, :nb] = torch.as_tensor(perm, dtype=torch.int32, device=DEV)
    return kc, vc, table


@pytest.mark.parametrize("N,bs,topk", [(1000, 16, 128), (5000, 64, 500), (20001, 128, 2048)])
def test_paged_anchor_decode(N, bs, topk):
    say("paged anchor decode", N, bs, topk)
    cfg = configs.LLAMA_DECODE_32K
    lin = synth.heavy_lineages(cfg.seed, 1, 2, N, max(1, N // 10), cfg.drift)
    q, k, v = synth.decode_layer(cfg.seed, 0, 2, 8, 2, 128, N, lin[0], cfg.alpha, "bf16", device=DEV)
    kc, vc, table = _paged(k, v, bs, seed=N)
    out, lse, idx, pooled = K.anchor_decode_paged(q, kc, vc, table, N, topk, want_pooled=True)
    torch.cuda.synchronize()
    ro, rl, rpool, ridx = oracle.anchor_decode(np64(q), np64(k), np64(v), topk)
    assert np.max(np.abs(np64(out) - ro)) <= 2e-2
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-4
    gp = np64(pooled)
    assert np.max(np.abs(gp - rpool) / np.maximum(rpool, 1e-30)) < 1e-4 or np.max(np.abs(gp - rpool)) < 1e-6
    gi = idx.cpu().numpy()
    for b in range(gi.shape[0]):
        for g in range(gi.shape[1]):
            assert np.array_equal(gi[b, g], oracle.topk_full_sort(gp[b, g], topk))
            ok, nd = oracle.index_sets_agree(gi[b, g], ridx[b, g], rpool[b, g])
            assert ok, (b, g, nd)


@pytest.mark.parametrize("N,bs,topk,hm", [(3000, 16, 300, [1, 0]), (9000, 256, 900, [1, 1])])
def test_paged_reuse_decode(N, bs, topk, hm):
    say("paged reuse decode", N, bs, topk, hm)
    g = torch.Generator(device=DEV).manual_seed(N)
    q = torch.randn((2, 8, 128), generator=g, device=DEV).bfloat16()
    k = torch.randn((2, 2, N, 128), generator=g, device=DEV).bfloat16()
    v = torch.randn((2, 2, N, 128), generator=g, device=DEV).bfloat16()
    idx = synth.random_index_lists(N + topk, 2, 2, N, topk, device=DEV)
    kc, vc, table = _paged(k, v, bs, seed=N + 1)
    out = K.reuse_decode_paged(q, kc, vc, table, N, idx, hm)
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_decode(np64(q), np64(k), np64(v), idx.cpu().numpy(), hm)
    assert np.max(np.abs(np64(out) - ref)) <= 2e-2
    # the contiguous path on the same logical cache agrees to rounding
    out_c = K.reuse_decode(q, k, v, idx, hm)
    torch.cuda.synchronize()
    assert np.max(np.abs(np64(out) - np64(out_c))) <= 1e-2


def _tile_lists(seed, B, T, Hkv, N):
    """Seeded prefill tile lists [B,T,Hkv,k_max]: k_t ascending distinct
    positions below P_t per (batch, tile, KV head), -1 padded."""
    kmax = oracle.prefill_tile_k(T - 1, N)[1]
    rng = np.random.default_rng(seed)
    out = -np.ones((B, T, Hkv, kmax), dtype=np.int32)
    for b in range(B):
        for t in range(T):
            P, kt = oracle.prefill_tile_k(t, N)
            for g in range(Hkv):
                out[b, t, g, :kt] = np.sort(rng.choice(P, size=kt, replace=False))
    return out


@pytest.mark.parametrize("B,Hq,Hkv,N,bs,hm", [
    (1, 8, 2, 1000, 16, [1, 0]),          # ragged last block and tile, swapped heads
    (2, 8, 2, 2049, 64, [1, 1]),          # two batches, many-to-one map, one-row last tile
    (1, 16, 4, 3000, 32, [3, 0, 0, 2]),   # group of 4
    (1, 2, 2, 600, 128, [1, 0]),          # group of 1 (the four-wave kernel)
])
def test_paged_reuse_prefill(B, Hq, Hkv, N, bs, hm):
    say("paged reuse prefill", B, Hq, Hkv, N, bs, hm)
    g = torch.Generator(device=DEV).manual_seed(N + bs)
    q = torch.randn((B, Hq, N, 128), generator=g, device=DEV).bfloat16()
    k = torch.randn((B, Hkv, N, 128), generator=g, device=DEV).bfloat16()
    v = torch.randn((B, Hkv, N, 128), generator=g, device=DEV).bfloat16()
    T = -(-N // 128)
    lists = _tile_lists(N + 3, B, T, Hkv, N)
    idx = torch.as_tensor(lists, device=DEV)
    kc, vc, table = _paged(k, v, bs, seed=N + 2)
    out = K.reuse_prefill_paged(q, kc, vc, table, idx, hm)
    out_c = K.reuse_prefill(q, k, v, idx, hm)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    qn, kn, vn, on = np64(q), np64(k), np64(v), np64(out)
    rows = sorted({0, 1, 127, 128, N // 2, N - 2, N - 1})
    for b in {0, B - 1}:
        for h in {0, Hq // 2, Hq - 1}:
            ref = oracle.sparse_prefill_rows(qn, kn, vn, lists, hm, b, h, rows)
            assert np.max(np.abs(on[b, h, rows] - ref)) <= 2e-2, (b, h)


def test_paged_reuse_prefill_longest_list():
    """The longest list the paged reuse prefill stages (12288 keys: positions
    and physical rows both sit in LDS): k_t the whole prefix (pct 100), so
    the output is dense causal attention; bitwise the contiguous pass, and
    against the oracle on sampled rows."""
    N, Hq, Hkv, bs = 12288, 2, 1, 64
    say("paged reuse prefill longest list", N, bs)
    g = torch.Generator(device=DEV).manual_seed(31)
    q = torch.randn((1, Hq, N, 128), generator=g, device=DEV).bfloat16()
    k = torch.randn((1, Hkv, N, 128), generator=g, device=DEV).bfloat16()
    v = torch.randn((1, Hkv, N, 128), generator=g, device=DEV).bfloat16()
    rule = K.TopkRule(128, 100, 64, 256)
    kmax = K.kascade_topk_for_len(N, rule)
    assert kmax == 12288
    T = N // 128
    lists = -np.ones((1, T, Hkv, kmax), dtype=np.int32)
    for t in range(T):
        lists[0, t, 0, :128 * (t + 1)] = np.arange(128 * (t + 1))
    idx = torch.as_tensor(lists, device=DEV)
    kc, vc, table = _paged(k, v, bs, seed=33)
    out = K.reuse_prefill_paged(q, kc, vc, table, idx, [0], rule)
    out_c = K.reuse_prefill(q, k, v, idx, [0], rule)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    qn, kn, vn, on = np64(q), np64(k), np64(v), np64(out)
    rows = [0, 1, 127, 128, 5000, N - 1]
    for h in range(Hq):
        ro, _, _ = oracle.dense_prefill_rows(qn, kn, vn, 0, h, rows)
        assert np.max(np.abs(on[0, h, rows] - ro)) <= 2e-2, h


def test_paged_reuse_prefill_32k():
    """Full-size reuse layer of the 32K-token prompt workload (32 q / 8 KV
    heads, bf16, block size 16, blocks scattered): bit-identical to the
    contiguous call (which the 32K prefill test checks against the oracle),
    and the oracle checks sampled rows of two tiles directly."""
    cfg = configs.LLAMA_PREFILL_32K
    N, Hkv, d, bs = cfg.ctx_len, cfg.n_kv_heads, cfg.head_dim, 16
    say("paged reuse prefill 32K", N, bs)
    lin = synth.heavy_lineages(cfg.seed, 2, Hkv, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, 2, (0,), Hkv, cfg.head_map_kind)
    q, k, v = synth.prefill_layer(cfg.seed, 1, 1, cfg.n_q_heads, Hkv, d, N,
                                  synth.layer_heavy_sets(lin, 1, (0,), maps), cfg.alpha, cfg.gamma, "bf16",
                                  device=DEV)
    T = N // 128
    lists = _tile_lists(cfg.seed, 1, T, Hkv, N)
    idx = torch.as_tensor(lists, device=DEV)
    kc, vc, table = _paged(k, v, bs, seed=cfg.seed)
    out = K.reuse_prefill_paged(q, kc, vc, table, idx, maps[1])
    out_c = K.reuse_prefill(q, k, v, idx, maps[1])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
    qn, kn, vn = np64(q), np64(k), np64(v)
    for t in (3, T - 1):
        rows = [128 * t, 128 * t + 77, 128 * t + 127]
        for h in (0, cfg.n_q_heads - 1):
            ref = oracle.sparse_prefill_rows(qn, kn, vn, lists, maps[1], 0, h, rows)
            assert np.max(np.abs(np64(out[0, h, rows]) - ref)) <= 2e-2, (t, h)


def _paged_fast(k, v, bs, seed):
    """Vectorised _paged for large caches (N a multiple of bs, no spare blocks)."""
    B, Hkv, N, d = k.shape
    nb = N // bs
    perm = torch.as_tensor(np.random.default_rng(seed).permutation(B * nb).reshape(B, nb), dtype=torch.int64,
                           device=DEV)
    kc = torch.empty((B * nb, Hkv, bs, d), dtype=k.dtype, device=DEV)
    vc = torch.empty_like(kc)
    kc[perm.reshape(-1)] = k.view(B, Hkv, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, d)
    vc[perm.reshape(-1)] = v.view(B, Hkv, nb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, d)
    return kc, vc, perm.to(torch.int32).contiguous()


def test_paged_decode_128k_sampled():
    """Full-size paged anchor and reuse decode of the 128K x 4 workload (block
    size 16, blocks scattered); the oracle checks batch row 2 and KV heads 1
    and 7 on the logical caches."""
    cfg = configs.LLAMA_DECODE_128K
    N, B, Hkv, G, k = cfg.ctx_len, cfg.batch, cfg.n_kv_heads, cfg.group, cfg.topk
    say("paged decode 128K x 4, sampled rows")
    lin = synth.heavy_lineages(cfg.seed, 2, Hkv, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, 2, (0,), Hkv, cfg.head_map_kind)
    q, kk, v = synth.decode_layer(cfg.seed, 0, B, cfg.n_q_heads, Hkv, cfg.head_dim, N,
                                  synth.layer_heavy_sets(lin, 0, (0,), maps), cfg.alpha, "bf16", device=DEV)
    kc, vc, table = _paged_fast(kk, v, 16, seed=5)
    out, _, idx, pooled = K.anchor_decode_paged(q, kc, vc, table, N, k, want_pooled=True)
    q1, k1, v1 = synth.decode_layer(cfg.seed, 1, B, cfg.n_q_heads, Hkv, cfg.head_dim, N,
                                    synth.layer_heavy_sets(lin, 1, (0,), maps), cfg.alpha, "bf16", device=DEV)
    kc1, vc1, table1 = _paged_fast(k1, v1, 16, seed=6)
    hm = maps[1]
    out1 = K.reuse_decode_paged(q1, kc1, vc1, table1, N, idx, hm)
    torch.cuda.synchronize()
    b = 2
    for g in (1, 7):
        hs = slice(g * G, (g + 1) * G)
        ro, _, p = oracle.dense_decode(np64(q[b:b + 1, hs]), np64(kk[b:b + 1, g:g + 1]), np64(v[b:b + 1, g:g + 1]))
        assert np.max(np.abs(np64(out[b:b + 1, hs]) - ro)) <= 2e-2
        rpool = oracle.pool_decode(p, 1)[0, 0]
        ridx = oracle.topk_full_sort(rpool, k)
        gi = idx[b, g].cpu().numpy()
        assert np.array_equal(gi, oracle.topk_full_sort(np64(pooled[b, g]), k))
        ok, nd = oracle.index_sets_agree(gi, ridx, rpool)
        assert ok, (g, nd)
        for g2 in [x for x in range(Hkv) if hm[x] == g]:
            hs2 = slice(g2 * G, (g2 + 1) * G)
            r1, _ = oracle.sparse_decode(np64(q1[b:b + 1, hs2]), np64(k1[b:b + 1, g2:g2 + 1]),
                                         np64(v1[b:b + 1, g2:g2 + 1]), ridx[None, None, :], [0])
            assert np.max(np.abs(np64(out1[b:b + 1, hs2]) - r1)) <= 2e-2

"""Seeded random-shape sweep of the four entry points against the oracle.

Each case draws its shape from a fixed seed: batch, KV heads, query-group
size, context or prompt length (log-uniform or uniform over a range,
ragged), Top-k (decode), dtype (fp32 with d 64, bf16 or fp16 with d 128)
and a random many-to-one head map.
Anchor layers are checked in full (outputs, lse, pooled values, index
lists; 16-bit cases also through the one-launch anchor decode, bit for bit
against the four-launch call); reuse layers run on the ORACLE's index lists,
so both sides consume the same lists.  16-bit cases also run over paged caches (random block size,
blocks scattered): paged decode against the oracle, paged reuse prefill bit
for bit against the contiguous call.  Tolerances as in the other GPU tests: outputs 1e-4 (fp32) /
2e-2 (16-bit) max-abs, decode lse 1e-4, prefill lse 1e-3, pooled 1e-4
(decode) / 1e-3 (prefill tile rows) relative, index sets bit-exact against a
full sort of the GPU's own pooled row and within the 1e-5 tie band of the
oracle's."""
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_anchor_amd import synth
from long_context_anchor_amd import kascade as K
from test_gpu_paged import _paged

pytestmark = pytest.mark.gpu
DEV = "cuda"
RULE = K.PREFILL_RULE


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _decode_case(seed):
    r = np.random.default_rng(1000 + seed)
    dtype = ["f32", "bf16", "f16"][seed % 3]
    d = 64 if dtype == "f32" else 128
    B = int(r.integers(1, 4))
    Hkv = int(r.choice([1, 2, 3, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    # even seeds: log-uniform lengths (many tiny, ragged ones); odd: 1000..6000
    N = int(np.exp(r.uniform(0.0, np.log(6000.0)))) if seed % 2 == 0 else int(r.integers(1000, 6001))
    N = max(N, 1)
    topk = int(r.integers(1, N + 1))
    hm = [int(x) for x in r.integers(0, Hkv, size=Hkv)]
    return dtype, d, B, Hkv, G, N, topk, hm


def _prefill_case(seed):
    r = np.random.default_rng(2000 + seed)
    dtype = ["bf16", "f16"][(seed // 2) % 2]
    B = int(r.integers(1, 3))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4]))
    N = int(np.exp(r.uniform(0.0, np.log(1200.0)))) if seed % 2 == 0 else int(r.integers(300, 1201))
    N = max(N, 1)
    hm = [int(x) for x in r.integers(0, Hkv, size=Hkv)]
    return dtype, B, Hkv, G, N, hm


def _randn(shape, seed, dtype):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(synth.torch_dtype(dtype))


@pytest.mark.parametrize("seed", range(40))
def test_random_decode(seed):
    dtype, d, B, Hkv, G, N, topk, hm = _decode_case(seed)
    Hq = G * Hkv
    say("random decode", seed, dtype, "B", B, "Hq", Hq, "Hkv", Hkv, "N", N, "k", topk, "hm", hm)
    tol = 1e-4 if dtype == "f32" else 2e-2
    # anchor layer: keys with a planted heavy set so the pooled rows are not flat
    lin = synth.heavy_lineages(seed, 2, Hkv, N, max(1, N // 10), 0.1)
    q, k, v = synth.decode_layer(seed, 0, B, Hq, Hkv, d, N, lin[0], 3.0, dtype, device=DEV)
    out, lse, idx, pooled = K.anchor_decode(q, k, v, topk, want_pooled=True)
    torch.cuda.synchronize()
    ro, rl, rpool, ridx = oracle.anchor_decode(np64(q), np64(k), np64(v), topk)
    assert np.max(np.abs(np64(out) - ro)) <= tol
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-4
    gp = np64(pooled)
    assert np.max(np.abs(gp - rpool) / np.maximum(rpool, 1e-30)) < 1e-4 or np.max(np.abs(gp - rpool)) < 1e-6
    gi = idx.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            assert np.all(np.diff(gi[b, g]) > 0)
            assert np.array_equal(gi[b, g], oracle.topk_full_sort(gp[b, g], topk))
            ok, nd = oracle.index_sets_agree(gi[b, g], ridx[b, g], rpool[b, g])
            assert ok, (b, g, nd)
    if dtype != "f32":
        # the one-launch anchor decode: bit for bit the four-launch outputs
        fo, fl, fi, fpool = K.anchor_decode_fused(q, k, v, topk, want_pooled=True)
        torch.cuda.synchronize()
        assert torch.equal(fo.view(torch.int16), out.view(torch.int16))
        assert torch.equal(fl, lse) and torch.equal(fi, idx) and torch.equal(fpool, pooled)
    # reuse layer on the oracle's lists through a random head map
    q2 = _randn((B, Hq, d), 7 * seed + 1, dtype)
    k2 = _randn((B, Hkv, N, d), 7 * seed + 2, dtype)
    v2 = _randn((B, Hkv, N, d), 7 * seed + 3, dtype)
    lists = torch.as_tensor(np.ascontiguousarray(ridx, dtype=np.int32), device=DEV)
    o2 = K.reuse_decode(q2, k2, v2, lists, hm)
    torch.cuda.synchronize()
    r2, _ = oracle.sparse_decode(np64(q2), np64(k2), np64(v2), ridx, hm)
    assert np.max(np.abs(np64(o2) - r2)) <= tol
    if dtype == "f32":
        return   # paged caches are 16-bit only
    # the same two layers over paged caches (random block size, blocks scattered)
    bs = int(np.random.default_rng(3000 + seed).choice([16, 32, 64, 128]))
    kc, vc, table = _paged(k, v, bs, seed=seed)
    po, _, pidx, ppool = K.anchor_decode_paged(q, kc, vc, table, N, topk, want_pooled=True)
    kc2, vc2, table2 = _paged(k2, v2, bs, seed=seed + 1)
    po2 = K.reuse_decode_paged(q2, kc2, vc2, table2, N, lists, hm)
    torch.cuda.synchronize()
    assert np.max(np.abs(np64(po) - ro)) <= tol
    gpp, gpi = np64(ppool), pidx.cpu().numpy()
    for b in range(B):
        for g in range(Hkv):
            assert np.array_equal(gpi[b, g], oracle.topk_full_sort(gpp[b, g], topk))
            ok, nd = oracle.index_sets_agree(gpi[b, g], ridx[b, g], rpool[b, g])
            assert ok, ("paged", b, g, nd)
    assert np.max(np.abs(np64(po2) - r2)) <= tol


@pytest.mark.parametrize("seed", range(16))
def test_random_prefill(seed):
    dtype, B, Hkv, G, N, hm = _prefill_case(seed)
    Hq = G * Hkv
    say("random prefill", seed, dtype, "B", B, "Hq", Hq, "Hkv", Hkv, "N", N, "hm", hm)
    lin = synth.heavy_lineages(seed, 1, Hkv, N, max(1, N // 10), 0.05)
    q, k, v = synth.prefill_layer(seed, 0, B, Hq, Hkv, 128, N, lin[0], 3.0, 4.0, dtype, device=DEV)
    out, lse, idx, pooled = K.anchor_prefill(q, k, v, RULE, want_pooled=True)
    torch.cuda.synchronize()
    qn, kn, vn = np64(q), np64(k), np64(v)
    gidx, gpool = idx.cpu().numpy(), pooled.cpu().numpy()
    T = -(-N // 128)
    kmax = oracle.prefill_tile_k(T - 1, N)[1]
    lists = -np.ones((B, T, Hkv, kmax), dtype=np.int32)
    for b in range(B):
        for h in (0, Hq - 1):
            ro, rl, _ = oracle.dense_prefill_rows(qn, kn, vn, b, h, range(N))
            assert np.max(np.abs(np64(out[b, h]) - ro)) <= 2e-2
            assert np.max(np.abs(np64(lse[b, h]) - rl)) <= 1e-3
        for t in range(T):
            P, kt = oracle.prefill_tile_k(t, N)
            for g in range(Hkv):
                rp = oracle.tile_pool_one(qn, kn, b, t, g)
                gp = K.packed_row(torch.as_tensor(gpool[b]), t, g, N, Hkv).numpy().astype(np.float64)
                assert np.max(np.abs(gp - rp) / np.maximum(rp, 1e-6)) <= 1e-3
                row = gidx[b, t, g]
                assert np.all(row[kt:] == -1)
                assert np.array_equal(row[:kt], oracle.topk_full_sort(gp, kt))
                ri = oracle.topk_full_sort(rp, kt)
                ok, nd = oracle.index_sets_agree(row[:kt], ri, rp)
                assert ok, (b, t, g, nd)
                lists[b, t, g, :kt] = ri
    # reuse layer on the oracle's tile lists through a random head map
    q2 = _randn((B, Hq, N, 128), 11 * seed + 1, dtype)
    k2 = _randn((B, Hkv, N, 128), 11 * seed + 2, dtype)
    v2 = _randn((B, Hkv, N, 128), 11 * seed + 3, dtype)
    lists_d = torch.as_tensor(lists, device=DEV)
    o2 = K.reuse_prefill(q2, k2, v2, lists_d, hm, RULE)
    # over a paged cache (random block size, blocks scattered): the same rows
    # with the same arithmetic, so bit for bit the contiguous output
    bs = int(np.random.default_rng(4000 + seed).choice([16, 32, 64, 128]))
    kc2, vc2, table2 = _paged(k2, v2, bs, seed=seed)
    po2 = K.reuse_prefill_paged(q2, kc2, vc2, table2, lists_d, hm, RULE)
    torch.cuda.synchronize()
    assert torch.equal(po2.view(torch.int16), o2.view(torch.int16))
    q2n, k2n, v2n, o2n = np64(q2), np64(k2), np64(v2), np64(o2)
    rows = sorted({0, N // 3, N // 2, N - 1} | {min(N - 1, 128 * t + 127) for t in range(T)})
    for b in range(B):
        for h in (0, Hq // 2, Hq - 1):
            ref = oracle.sparse_prefill_rows(q2n, k2n, v2n, lists, hm, b, h, rows)
            assert np.max(np.abs(o2n[b, h, rows] - ref)) <= 2e-2, (b, h)

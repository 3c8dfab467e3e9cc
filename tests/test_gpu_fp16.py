"""GPU parity of the fp16 variants (decode and prefill, anchor and reuse
layers, contiguous and paged caches) against the fp64 oracle, through the C
ABI.  The kernels are the bf16 ones with fp16 element arithmetic (fp16 dot
products and MFMA, P rounded to fp16, fp32 accumulation), so the bf16
tolerances apply unchanged: outputs 2e-2 max-abs, decode lse 1e-4, prefill
lse 1e-3, pooled rows 1e-4 (decode) / 1e-3 (prefill) relative, indices
bit-exact against a full sort of the GPU's own pooled row and within the
1e-5 relative tie band of the oracle's."""
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_anchor_amd import configs, synth
from long_context_anchor_amd import kascade as K

pytestmark = pytest.mark.gpu
DEV = "cuda"
F16 = torch.float16


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _randn(gen, shape):
    return torch.randn(shape, generator=gen, device=DEV).to(F16)


def _check_anchor_decode(q, k, v, topk, res):
    out, lse, idx, pooled = res
    torch.cuda.synchronize()
    ro, rl, rpool, ridx = oracle.anchor_decode(np64(q), np64(k), np64(v), topk)
    assert out.dtype == F16
    assert np.max(np.abs(np64(out) - ro)) <= 2e-2
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-4
    gp = np64(pooled)
    assert np.max(np.abs(gp - rpool) / np.maximum(rpool, 1e-30)) < 1e-4 or \
        np.max(np.abs(gp - rpool)) < 1e-6
    gi = idx.cpu().numpy()
    for b in range(gi.shape[0]):
        for g in range(gi.shape[1]):
            assert np.array_equal(gi[b, g], oracle.topk_full_sort(gp[b, g], topk))
            ok, nd = oracle.index_sets_agree(gi[b, g], ridx[b, g], rpool[b, g])
            assert ok, (b, g, nd)


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 32, 8, 4099), (2, 16, 2, 70000)])
def test_fp16_dense_decode(B, Hq, Hkv, N):
    say("fp16 dense decode", B, Hq, Hkv, N)
    g = torch.Generator(device=DEV).manual_seed(N)
    q, k, v = _randn(g, (B, Hq, 128)), _randn(g, (B, Hkv, N, 128)), _randn(g, (B, Hkv, N, 128))
    out, lse = K.dense_decode(q, k, v)
    torch.cuda.synchronize()
    ro, rl, _ = oracle.dense_decode(np64(q), np64(k), np64(v))
    assert out.dtype == F16
    assert np.max(np.abs(np64(out) - ro)) <= 2e-2
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-4


@pytest.mark.parametrize("N,topk", [(1, 1), (1000, 128), (20000, 2048), (70001, 7000)])
def test_fp16_anchor_decode(N, topk):
    say("fp16 anchor decode", N, topk)
    cfg = configs.LLAMA_DECODE_32K
    lin = synth.heavy_lineages(cfg.seed, 1, 2, N, max(1, N // 10), cfg.drift)
    q, k, v = synth.decode_layer(cfg.seed, 0, 2, 8, 2, 128, N, lin[0], cfg.alpha, "f16", device=DEV)
    _check_anchor_decode(q, k, v, topk, K.anchor_decode(q, k, v, topk, want_pooled=True))


@pytest.mark.parametrize("G,N,topk,hm", [(4, 4096, 333, [2, 2, 0, 1]), (8, 10000, 1000, [1, 1]),
                                         (1, 777, 777, [0, 0])])
def test_fp16_reuse_decode(G, N, topk, hm):
    say("fp16 reuse decode", G, N, topk, hm)
    Hkv = len(hm)
    g = torch.Generator(device=DEV).manual_seed(N + topk)
    q, k, v = _randn(g, (2, G * Hkv, 128)), _randn(g, (2, Hkv, N, 128)), _randn(g, (2, Hkv, N, 128))
    idx = synth.random_index_lists(N + topk, 2, Hkv, N, topk, device=DEV)
    out = K.reuse_decode(q, k, v, idx, hm)
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_decode(np64(q), np64(k), np64(v), idx.cpu().numpy(), hm)
    assert out.dtype == F16
    assert np.max(np.abs(np64(out) - ref)) <= 2e-2


def test_fp16_paged_anchor_and_reuse_decode():
    N, bs, topk, hm = 5000, 64, 500, [1, 0]
    say("fp16 paged decode", N, bs, topk, hm)
    g = torch.Generator(device=DEV).manual_seed(77)
    q, k, v = _randn(g, (2, 8, 128)), _randn(g, (2, 2, N, 128)), _randn(g, (2, 2, N, 128))
    nb = -(-N // bs)
    perm = np.random.default_rng(5).permutation(2 * nb + 3)[: 2 * nb].reshape(2, nb)
    kc = torch.zeros((2 * nb + 3, 2, bs, 128), dtype=F16, device=DEV)
    vc = torch.zeros_like(kc)
    for b in range(2):
        for i in range(nb):
            lo, hi = i * bs, min(N, (i + 1) * bs)
            kc[perm[b, i], :, : hi - lo] = k[b, :, lo:hi]
            vc[perm[b, i], :, : hi - lo] = v[b, :, lo:hi]
    table = torch.as_tensor(perm, dtype=torch.int32, device=DEV)
    _check_anchor_decode(q, k, v, topk,
                         K.anchor_decode_paged(q, kc, vc, table, N, topk, want_pooled=True))
    idx = synth.random_index_lists(9, 2, 2, N, topk, device=DEV)
    out = K.reuse_decode_paged(q, kc, vc, table, N, idx, hm)
    torch.cuda.synchronize()
    ref, _ = oracle.sparse_decode(np64(q), np64(k), np64(v), idx.cpu().numpy(), hm)
    assert np.max(np.abs(np64(out) - ref)) <= 2e-2


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 2, 1, 128), (2, 4, 2, 200), (1, 16, 2, 257)])
def test_fp16_dense_prefill(B, Hq, Hkv, N):
    say("fp16 dense prefill", B, Hq, Hkv, N)
    g = torch.Generator(device=DEV).manual_seed(N + Hq)
    q, k, v = _randn(g, (B, Hq, N, 128)), _randn(g, (B, Hkv, N, 128)), _randn(g, (B, Hkv, N, 128))
    out, lse = K.dense_prefill(q, k, v)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_prefill(np64(q), np64(k), np64(v))
    assert out.dtype == F16
    assert np.max(np.abs(np64(out) - ro)) <= 2e-2
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-3


@pytest.mark.parametrize("B,Hq,Hkv,N,hm", [(1, 8, 2, 300, [1, 0]), (1, 16, 2, 1100, [1, 1]),
                                           (2, 4, 4, 640, [3, 0, 1, 2])])
def test_fp16_anchor_and_reuse_prefill(B, Hq, Hkv, N, hm):
    say("fp16 anchor+reuse prefill", B, Hq, Hkv, N, hm)
    cfg = configs.LLAMA_PREFILL_32K
    lin = synth.heavy_lineages(N, 1, Hkv, N, max(1, N // 10), cfg.drift)
    q, k, v = synth.prefill_layer(N, 0, B, Hq, Hkv, 128, N, lin[0], cfg.alpha, cfg.gamma, "f16",
                                  device=DEV)
    rule = K.PREFILL_RULE
    out, lse, idx, pooled = K.anchor_prefill(q, k, v, rule, want_pooled=True)
    torch.cuda.synchronize()
    assert out.dtype == F16
    qn, kn, vn = np64(q), np64(k), np64(v)
    ro, rl = oracle.dense_prefill(qn, kn, vn)
    assert np.max(np.abs(np64(out) - ro)) <= 2e-2
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-3
    T = -(-N // 128)
    gidx = idx.cpu().numpy()
    gpool = pooled.cpu().numpy()
    for b in range(B):
        for t in range(T):
            _, kt = oracle.prefill_tile_k(t, N)
            for g in range(Hkv):
                rp = oracle.tile_pool_one(qn, kn, b, t, g)
                gp = K.packed_row(torch.as_tensor(gpool[b]), t, g, N, Hkv).numpy().astype(np.float64)
                assert np.max(np.abs(gp - rp) / np.maximum(rp, 1e-6)) <= 1e-3
                sel = gidx[b, t, g, :kt]
                assert np.all(gidx[b, t, g, kt:] == -1)
                assert np.array_equal(sel, oracle.topk_full_sort(gp, kt))
                ok, nd = oracle.index_sets_agree(sel, oracle.topk_full_sort(rp, kt), rp)
                assert ok, (b, t, g, nd)
    # reuse layer over the anchor's lists, against the oracle on the same lists
    q2 = _randn(torch.Generator(device=DEV).manual_seed(N + 1), q.shape)
    out2 = K.reuse_prefill(q2, k, v, idx, hm, rule)
    torch.cuda.synchronize()
    ref = oracle.sparse_prefill(np64(q2), kn, vn, gidx, hm)
    assert out2.dtype == F16
    assert np.max(np.abs(np64(out2) - ref)) <= 2e-2

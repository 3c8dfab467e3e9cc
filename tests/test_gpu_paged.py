"""GPU parity of decode over paged KV caches (block tables, layout
[num_blocks, Hkv, block_size, d], blocks scattered by a seeded permutation,
ragged last block) against the oracle on the logical caches.  Tolerances as
for contiguous decode: outputs 2e-2 max-abs (bf16), lse 1e-4, pooled 1e-4
relative, indices bit-exact against a full sort of the GPU's own pooled row
and within the 1e-5 tie band of the oracle's."""
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

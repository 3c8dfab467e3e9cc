"""GPU parity of the calibration path: per-KV-head cross-layer similarity of
the anchor decode pass's pooled rows, the layer weight, and the whole flow
(similarities -> weighted similarity -> anchor DP -> head maps) against the
oracle's own flow.  Similarities within 1e-4 (fp32 pooled rows against fp64,
index sets equal up to near-ties); layer weight within 1e-5."""
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


def _stack(L, S, Hkv, G, N, k, seed, maps_kind="perm"):
    """L decode layers (S batch rows = calibration queries) with planted heavy
    keys drifting across layers; returns GPU pooled/idx stacks and the inputs."""
    anchors = (0,)
    lin = synth.heavy_lineages(seed, L, Hkv, N, max(1, N // 10), 0.05)
    maps = synth.head_maps(seed, L, anchors, Hkv, maps_kind)
    layers, pooled, idx = [], [], []
    for l in range(L):
        q, kk, v = synth.decode_layer(seed, l, S, G * Hkv, Hkv, 128, N,
                                      synth.layer_heavy_sets(lin, l, anchors, maps), 6.0, "bf16",
                                      device=DEV)
        _, _, ix, po = K.anchor_decode(q, kk, v, k, want_pooled=True)
        layers.append((q, kk, v))
        pooled.append(po)
        idx.append(ix)
    return layers, torch.stack(pooled), torch.stack(idx), maps


def test_head_similarity_parity():
    L, S, Hkv, G, N, k = 4, 3, 4, 2, 3000, 300
    say("calib head similarity", L, S, Hkv, N, k)
    layers, pooled, idx, _ = _stack(L, S, Hkv, G, N, k, seed=21)
    sim = K.calib_head_similarity(pooled, idx)
    torch.cuda.synchronize()
    gs = sim.cpu().numpy().astype(np.float64)
    rpool = []
    for q, kk, v in layers:
        _, _, rp, _ = oracle.anchor_decode(np64(q), np64(kk), np64(v), k)
        rpool.append(rp)
    for a in range(L):
        for b in range(a, L):
            want = oracle.head_similarity(rpool[a], rpool[b], k)
            assert np.max(np.abs(gs[a, b] - want)) <= 1e-4, (a, b)
    # a layer against itself: every head is its own best match, similarity 1
    for a in range(L):
        assert np.max(np.abs(np.diag(gs[a, a]) - 1.0)) <= 1e-6


def test_calibration_flow_matches_oracle():
    """Similarities, layer weights, anchors by the DP, head maps: the library's
    flow on the GPU's pooled rows against the oracle's flow on its own."""
    L, S, Hkv, G, N, k, M = 6, 2, 4, 2, 2048, 256, 3
    say("calibration flow", L, M)
    layers, pooled, idx, maps = _stack(L, S, Hkv, G, N, k, seed=22)
    sim = K.calib_head_similarity(pooled, idx).cpu().numpy()
    g = torch.Generator(device=DEV).manual_seed(5)
    xs = [torch.randn((64, 256), generator=g, device=DEV) for _ in range(L)]
    ys = [x + (0.2 + 0.3 * l) * torch.randn((64, 256), generator=g, device=DEV) for l, x in enumerate(xs)]
    w = np.array([K.layer_weight(x, y).item() for x, y in zip(xs, ys)], dtype=np.float32)
    S_lib = K.kascade_weighted_similarity(L, Hkv, sim, w)
    anchors, _ = K.kascade_select_anchors(L, M, S_lib)
    hm = K.kascade_head_maps(L, Hkv, sim, anchors)

    rpool = []
    for q, kk, v in layers:
        _, _, rp, _ = oracle.anchor_decode(np64(q), np64(kk), np64(v), k)
        rpool.append(rp)
    rw = np.array([oracle.layer_weight(np64(x), np64(y)) for x, y in zip(xs, ys)])
    assert np.max(np.abs(w - rw)) <= 1e-5
    sbar = np.zeros((L, L))
    rsim = {}
    for a in range(L):
        for b in range(a, L):
            rsim[a, b] = oracle.head_similarity(rpool[a], rpool[b], k)
            sbar[a, b] = oracle.remapped_layer_similarity(rsim[a, b])
    S_ref = oracle.weighted_similarity(sbar, rw)
    assert np.max(np.abs(S_lib - S_ref)) <= 1e-4
    ranchors, _ = oracle.dp_select_anchors(S_ref, M)
    assert anchors == ranchors
    for b in range(L):
        a = oracle.anchor_of(b, anchors)
        if a != b:
            assert list(hm[b]) == list(oracle.head_map_from_similarity(rsim[a, b])), b
    # the planted structure: a reuse head's heavy keys come from anchor head
    # maps[b][gb] when the anchor is layer 0, and the calibration finds it
    for b in range(1, anchors[1] if len(anchors) > 1 else L):
        assert list(hm[b]) == [int(x) for x in maps[b]], b


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_layer_weight_parity(dtype):
    g = torch.Generator(device=DEV).manual_seed(9)
    x = torch.randn((1000, 512), generator=g, device=DEV)
    y = 0.7 * x + 0.5 * torch.randn((1000, 512), generator=g, device=DEV)
    x, y = x.to(dtype), y.to(dtype)
    w = K.layer_weight(x, y).item()
    assert abs(w - oracle.layer_weight(np64(x), np64(y))) <= 1e-5
    y[3].zero_()
    assert np.isnan(K.layer_weight(x, y).item())

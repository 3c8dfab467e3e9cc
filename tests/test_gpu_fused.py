"""GPU parity of the one-launch anchor decode (kascade_anchor_decode_fused),
through the C ABI, against the fp64 oracle and against the four-launch
anchor decode (kascade_anchor_decode).

Both paths take the same split plan and run the same arithmetic per split,
lse, pooled key and select step, so their outputs, lse, pooled rows and
lists must be bitwise equal.  Against the oracle the tolerances are those of
the anchor decode tests: outputs max-abs 2e-2 (16-bit inputs), lse 1e-4,
pooled rows 1e-4 relative, lists bit-exact against a full sort of the GPU's
own pooled row and within the oracle's 1e-5 tie band.
"""
import dataclasses
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


def _layer(cfg, layer, n=None, batch=None, n_kv=None, group=None):
    n = n or cfg.ctx_len
    B = batch or cfg.batch
    Hkv = n_kv or cfg.n_kv_heads
    G = group or cfg.group
    lin = synth.heavy_lineages(cfg.seed, max(layer + 1, 2), Hkv, n,
                               cfg.n_heavy or int(round(cfg.heavy_frac * n)), cfg.drift)
    maps = synth.head_maps(cfg.seed, max(layer + 1, 2), cfg.anchors, Hkv, cfg.head_map_kind)
    heavy = synth.layer_heavy_sets(lin, layer, cfg.anchors, maps)
    return synth.decode_layer(cfg.seed, layer, B, G * Hkv, Hkv, cfg.head_dim, n, heavy, cfg.alpha,
                              cfg.dtype, device=DEV)


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def _fused_equals_unfused(q, k, v, topk, ws=None, max_polls=0):
    """Runs both paths; asserts bitwise equality; returns the fused outputs."""
    f = K.anchor_decode_fused(q, k, v, topk, want_pooled=True, ws=ws, max_polls=max_polls)
    u = K.anchor_decode(q, k, v, topk, want_pooled=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("out", "lse", "idx", "pooled"), f, u):
        assert torch.equal(_bits(a), _bits(b)), name
    return f


def _check_oracle(q, k, v, topk, res, tol=2e-2):
    out, lse, idx, pooled = res
    ro, rl, rpool, ridx = oracle.anchor_decode(np64(q), np64(k), np64(v), topk)
    assert np.max(np.abs(np64(out) - ro)) <= tol
    assert np.max(np.abs(np64(lse) - rl)) <= 1e-4
    gp = np64(pooled)
    assert np.max(np.abs(gp - rpool) / np.maximum(rpool, 1e-30)) < 1e-4 or \
        np.max(np.abs(gp - rpool)) < 1e-6
    gi = idx.cpu().numpy()
    for b in range(gi.shape[0]):
        for g in range(gi.shape[1]):
            assert np.all(np.diff(gi[b, g]) > 0), "indices ascending and distinct"
            assert np.array_equal(gi[b, g], oracle.topk_full_sort(gp[b, g], topk))
            ok, nd = oracle.index_sets_agree(gi[b, g], ridx[b, g], rpool[b, g])
            assert ok, (b, g, nd)


@pytest.mark.parametrize("N,topk,B,Hkv,G,dtype", [
    (1, 1, 2, 2, 4, "bf16"), (130, 129, 2, 2, 4, "bf16"), (1000, 128, 2, 2, 4, "bf16"),
    (5000, 4999, 2, 2, 4, "bf16"), (20000, 2048, 2, 2, 4, "bf16"), (3000, 300, 1, 4, 1, "f16"),
    (9001, 1234, 2, 2, 8, "f16"), (4100, 4100, 1, 2, 2, "bf16"), (12345, 1500, 3, 2, 2, "f16"),
])
def test_fused_ragged_and_groups(N, topk, B, Hkv, G, dtype):
    cfg = dataclasses.replace(configs.LLAMA_DECODE_32K, dtype=dtype)
    say("fused anchor decode", N, topk, B, Hkv, G, dtype)
    q, k, v = _layer(cfg, 0, n=N, batch=B, n_kv=Hkv, group=G)
    res = _fused_equals_unfused(q, k, v, topk)
    _check_oracle(q, k, v, topk, res)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fused_llama_32k_layer(dtype):
    """The full 32K-context anchor layer of the Llama-shaped decode (one round
    of 256 workgroups: 8 KV heads x 32 splits of 1024 keys)."""
    cfg = dataclasses.replace(configs.LLAMA_DECODE_32K, dtype=dtype)
    say("fused 32K anchor layer", dtype)
    q, k, v = _layer(cfg, 0)
    res = _fused_equals_unfused(q, k, v, cfg.topk)
    _check_oracle(q, k, v, cfg.topk, res, cfg.tol)


def test_fused_64k_step():
    """A first decode step of the Qwen3-shaped 64K workload: 65537 keys, the
    decode k rule, 32 query and 8 KV heads (one round of 256 workgroups of
    2064 keys)."""
    cfg = configs.LLAMA_DECODE_32K
    n = configs.QWEN3_E2E_64K.ctx_len + 1
    topk = K.kascade_topk_for_len(n, K.DECODE_RULE)
    say("fused 64K step", n, topk)
    q, k, v = _layer(cfg, 0, n=n, batch=1)
    res = _fused_equals_unfused(q, k, v, topk)
    _check_oracle(q, k, v, topk, res)


def test_fused_constant_rows_take_the_first_positions():
    """A zero query gives every key the same pooled value: all keys tie and
    the list is the first topk positions."""
    g = torch.Generator(device=DEV).manual_seed(5)
    q = torch.zeros((1, 8, 128), device=DEV).bfloat16()
    k = torch.randn((1, 2, 30000, 128), generator=g, device=DEV).bfloat16()
    v = torch.randn((1, 2, 30000, 128), generator=g, device=DEV).bfloat16()
    _, _, idx, _ = _fused_equals_unfused(q, k, v, 3000)
    want = np.broadcast_to(np.arange(3000, dtype=np.int32), idx.shape)
    assert np.array_equal(idx.cpu().numpy(), want)


def _sync_words(ws, sh):
    """The workspace's row barrier counters (256 rows x 64 words after the status word)."""
    return ws[256:256 + 256 * 64 * 4].view(torch.int32)


def test_fused_repeated_calls_share_one_workspace():
    """Calls of different shapes in a row on one workspace: the status word
    stays zero and every call leaves the row counters zero."""
    cfg = configs.LLAMA_DECODE_32K
    big = _layer(cfg, 0)
    sh = K.make_shape(big[0], big[1], cfg.ctx_len)
    ws = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh, cfg.topk)
    for n, topk, B, Hkv in ((cfg.ctx_len, cfg.topk, 1, 8), (5000, 500, 1, 8), (20000, 2048, 1, 4),
                            (cfg.ctx_len, cfg.topk, 1, 8)):
        say("repeat", n, topk, B, Hkv)
        q, k, v = big if n == cfg.ctx_len else _layer(cfg, 0, n=n, batch=B, n_kv=Hkv)
        _fused_equals_unfused(q, k, v, topk, ws=ws)
        assert K.fused_status(ws) == 0
        assert int(_sync_words(ws, sh).abs().sum().item()) == 0


def test_fused_early_give_up_leaves_workspace_usable():
    """Failure handling, forced from the host: with at most one repeated poll
    per barrier most workgroups give up waiting, set the status bit and skip
    their remaining phases; the launch still ends normally, the counters are
    left zero, and the next call on the workspace is correct."""
    cfg = configs.LLAMA_DECODE_32K
    q, k, v = _layer(cfg, 0)
    sh = K.make_shape(q, k, cfg.ctx_len)
    ws = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh, cfg.topk)
    K.anchor_decode_fused(q, k, v, cfg.topk, ws=ws, max_polls=1)
    torch.cuda.synchronize()
    st = K.fused_status(ws)
    say("status after a one-poll call", st)
    assert st in (0, 1)
    assert int(_sync_words(ws, sh).abs().sum().item()) == 0
    ws[0:4].zero_()
    _fused_equals_unfused(q, k, v, cfg.topk, ws=ws)
    assert K.fused_status(ws) == 0


def test_fused_graph_replays_match_eager():
    """The call captured in a HIP graph (no memset nodes): several replays,
    with eager work and synchronisations between them, each equal to the
    eager result."""
    cfg = configs.LLAMA_DECODE_32K
    q, k, v = _layer(cfg, 0)
    sh = K.make_shape(q, k, cfg.ctx_len)
    ws = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh, cfg.topk)
    want = K.anchor_decode_fused(q, k, v, cfg.topk, ws=ws)
    torch.cuda.synchronize()
    B, Hq, d = q.shape
    out = torch.empty_like(want[0])
    lse = torch.empty_like(want[1])
    idx = torch.empty_like(want[2])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            K.check(K.kascade_anchor_decode_fused(sh, q, k, v, cfg.topk, out, lse, idx, None, 0, ws,
                                                  ws.numel(), s.cuda_stream), "fused capture")
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(0)
        idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say("replay", rep)
        assert torch.equal(_bits(out), _bits(want[0]))
        assert torch.equal(lse, want[1])
        assert torch.equal(idx, want[2])
        assert K.fused_status(ws) == 0


def test_fused_rejects_launches_that_cannot_be_resident():
    """128K x 4 needs more workgroups than the GPU holds at once (and splits
    whose scores do not fit in LDS): the call returns KASCADE_ERR_SHAPE
    without launching anything."""
    q = torch.zeros((4, 32, 128), device=DEV).bfloat16()
    k = torch.zeros((4, 8, 131072, 128), device=DEV).bfloat16()
    sh = K.make_shape(q, k, 131072)
    ws = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh, 13120)
    out = torch.full((4, 32, 128), 7, device=DEV).bfloat16()
    idx = torch.full((4, 8, 13120), -3, dtype=torch.int32, device=DEV)
    st = K.kascade_anchor_decode_fused(sh, q, k, k, 13120, out, None, idx, None, 0, ws, ws.numel())
    assert st == K.KASCADE_ERR_SHAPE
    torch.cuda.synchronize()
    assert int((idx != -3).sum().item()) == 0


def test_fused_many_calls_stay_bitwise_equal():
    """200 calls on one workspace, alternating two 32K anchor layers, each
    output compared bit for bit with the four-launch reference: the
    exchanged words (partials, histograms, candidates, counters) are seen
    complete in every call, and every call leaves the counters zero."""
    cfg = configs.LLAMA_DECODE_32K
    lays = [_layer(cfg, 0), _layer(cfg, 2)]
    refs = [K.anchor_decode(*x, cfg.topk) for x in lays]
    sh = K.make_shape(lays[0][0], lays[0][1], cfg.ctx_len)
    ws = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh, cfg.topk)
    out = torch.empty_like(refs[0][0])
    lse = torch.empty_like(refs[0][1])
    idx = torch.empty_like(refs[0][2])
    bad = 0
    for i in range(200):
        q, k, v = lays[i % 2]
        K.check(K.kascade_anchor_decode_fused(sh, q, k, v, cfg.topk, out, lse, idx, None, 0, ws, ws.numel()),
                "fused")
        ro, rl, ri, _ = refs[i % 2]
        ok = torch.equal(_bits(out), _bits(ro)) and torch.equal(lse, rl) and torch.equal(idx, ri)
        bad += 0 if ok else 1
    torch.cuda.synchronize()
    say("mismatching calls", bad, "of 200")
    assert bad == 0
    assert K.fused_status(ws) == 0
    assert int(_sync_words(ws, sh).abs().sum().item()) == 0

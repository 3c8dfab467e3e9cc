#!/usr/bin/env python3
"""Benchmark of the Kascade anchor/reuse Top-k attention hot path on one GPU.

One step = one pass of the whole hot path over the Llama-3.1-8B-shaped
synthetic workloads (32 layers, 32 query / 8 KV heads, head_dim 128, bf16,
anchors [0, 2, 8, 13, 14], random permutation head maps):
  * decode at context 32768, batch 1, k = 3264   (anchor + reuse decode)
  * decode at context 131072, batch 4, k = 13120 (anchor + reuse decode)
  * prefill of a 32768-token prompt, 128-query tiles, per-tile k (min 256)
All inputs are resident in HBM before timing starts; every layer has its own
KV buffers so the 256 MB last-level cache cannot serve them across layers.

Prints ONE JSON line.  `value` is the decode attention time per layer at the
32K context (the first quantity of the metric); `components` carries the
128K decode figures (us/layer, GB/s) and the prefill TFLOP/s; `roofline`
describes the kernel with the largest share of the step time, measured with
HIP events on its launch stream inside the timed steps.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn µs/layer + HBM GB/s at 32k/128k ctx; prefill attn TFLOP/s"
HBM_PEAK_GBS = 8000.0
FUSED_ANCHOR = False   # --anchor-decode fused: the sections' anchor layers use the one-launch kernel
MFMA16_PEAK_TFLOPS = 2500.0  # dense bf16 and fp16 MFMA peak
# HBM traffic of the kernels, read by rocprofv3 counters and stored as text
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_kernels_llama8b.md")
CSRC = os.path.join(ROOT, "long_context_anchor_amd", "csrc")
KERNEL_SOURCES = {"prefill_flash": "prefill.hip", "prefill_pool": "prefill.hip",
                  "prefill_sparse": "prefill.hip", "decode_splitk": "decode.hip",
                  "decode_combine": "decode.hip", "decode_pool": "decode.hip",
                  "reuse_decode": "decode.hip", "topk_select": "select.hip",
                  "topk_select_wide_a": "select.hip", "topk_select_wide_b": "select.hip",
                  "anchor_fused": "decode.hip"}
COPY_BYTES = 1 << 30  # the calibration copy reads and writes this many bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workload construction (synthetic, seeded)
# ---------------------------------------------------------------------------

def decode_bytes(cfg):
    """Algorithmic HBM bytes of one decode layer (16-bit K/V and queries):
    (anchor, reuse, dense).  Anchor: every K and V row of the cache, the
    queries read and the output written, the list written; reuse: the listed
    K and V rows, the list read, queries and output; dense: cache, queries,
    output."""
    e = 2
    io = cfg.batch * cfg.n_q_heads * cfg.head_dim * e * 2 + cfg.batch * cfg.n_kv_heads * cfg.topk * 4
    anchor = 2 * cfg.batch * cfg.n_kv_heads * cfg.ctx_len * cfg.head_dim * e + io
    reuse = 2 * cfg.batch * cfg.n_kv_heads * cfg.topk * cfg.head_dim * e + io
    dense = 2 * cfg.batch * cfg.n_kv_heads * cfg.ctx_len * cfg.head_dim * e + \
        cfg.batch * cfg.n_q_heads * cfg.head_dim * e * 2
    return anchor, reuse, dense


def prefill_flops(cfg):
    """Algorithmic FLOPs of one causal prefill layer: (flash pass, pooling
    pass).  The flash pass does Q K^T and P V over the causal triangle
    (4 d Hq N (N+1) / 2), the pooling pass recomputes Q K^T (half of that);
    the waste of the diagonal blocks is not counted."""
    d, Hq, N = cfg.head_dim, cfg.n_q_heads, cfg.ctx_len
    return 4.0 * d * Hq * N * (N + 1) / 2, 2.0 * d * Hq * N * (N + 1) / 2


def build_decode(workload, torch, K, synth, configs, dtype="bf16"):
    cfg = dataclasses.replace(workload, dtype=dtype)
    N, L = cfg.ctx_len, cfg.n_layers
    lin = synth.heavy_lineages(cfg.seed, L, cfg.n_kv_heads, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, L, cfg.anchors, cfg.n_kv_heads, cfg.head_map_kind)
    layers = []
    for l in range(L):
        q, k, v = synth.decode_layer(cfg.seed, l, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads,
                                     cfg.head_dim, N, synth.layer_heavy_sets(lin, l, cfg.anchors, maps),
                                     cfg.alpha, cfg.dtype, device="cuda")
        layers.append((q, k, v))
    sh = K.make_shape(layers[0][0], layers[0][1], N)
    ws_a = K.workspace(K.OP_ANCHOR_DECODE, sh, cfg.topk)
    ws_r = K.workspace(K.OP_REUSE_DECODE, sh, cfg.topk)
    idx = {a: torch.empty((cfg.batch, cfg.n_kv_heads, cfg.topk), dtype=torch.int32, device="cuda")
           for a in cfg.anchors}
    out = torch.empty_like(layers[0][0])
    anchor_of = {l: max(a for a in cfg.anchors if a <= l) for l in range(L)}

    ws_d = K.workspace(K.OP_DENSE_DECODE, sh)
    lse = torch.empty(layers[0][0].shape[:2], dtype=torch.float32, device="cuda")
    # the one-launch anchor decode, where its workgroups fit on the GPU at once
    ws_f = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh, cfg.topk)
    a0 = cfg.anchors[0]
    st = K.kascade_anchor_decode_fused(sh, *layers[a0], cfg.topk, out, None, idx[a0], None, 0, ws_f,
                                       ws_f.numel())
    if st not in (K.KASCADE_OK, K.KASCADE_ERR_SHAPE):
        K.check(st, "anchor_decode_fused")
    fused_ok = st == K.KASCADE_OK

    def anchor(l, q, k, v, fused):
        if fused:
            K.check(K.kascade_anchor_decode_fused(sh, q, k, v, cfg.topk, out, None, idx[l], None, 0, ws_f,
                                                  ws_f.numel()), "anchor_decode_fused")
        else:
            K.check(K.kascade_anchor_decode(sh, q, k, v, cfg.topk, out, None, idx[l], None,
                                            ws_a, ws_a.numel()), "anchor_decode")

    def run(kind=None):
        if kind == "dense":   # the GPU's own dense decode on every layer (comparison)
            for q, k, v in layers:
                K.check(K.kascade_dense_decode(sh, q, k, v, out, lse, ws_d, ws_d.numel()), "dense_decode")
            return
        fused = kind == "anchor_fused" or (kind in (None, "anchor") and FUSED_ANCHOR and fused_ok)
        for l, (q, k, v) in enumerate(layers):
            if l in cfg.anchors:
                if kind in (None, "anchor", "anchor_fused"):
                    anchor(l, q, k, v, fused)
            elif kind in (None, "reuse"):
                K.check(K.kascade_reuse_decode(sh, q, k, v, cfg.topk, idx[anchor_of[l]], maps[l], out,
                                               ws_r, ws_r.numel()), "reuse_decode")

    n_anchor = len(cfg.anchors)
    n_reuse = L - n_anchor
    bytes_anchor, bytes_reuse, bytes_dense = decode_bytes(cfg)
    return dict(cfg=cfg, run=run, n_anchor=n_anchor, n_reuse=n_reuse, bytes_anchor=bytes_anchor,
                bytes_reuse=bytes_reuse, bytes_dense=bytes_dense, layers=layers, maps=maps, fused_ok=fused_ok)


def prefill_reuse_flops(torch, K, idx_by_anchor, anchor_of, maps, layers_reuse, N, n_kv, group, d):
    """4*d*sum_{h,r} |J_{h,r}| over the reuse layers, counted from the anchors' tile lists
    (J_{h,r} = the listed positions j <= r of row r's tile for KV head head_map[h // group])."""
    rule = K.PREFILL_RULE
    T = N // rule.tile
    dev = next(iter(idx_by_anchor.values())).device
    rows = torch.arange(N, device=dev, dtype=torch.int64).view(T, rule.tile)
    per_anchor = {}
    for a, ix in idx_by_anchor.items():
        cnt = torch.zeros(n_kv, dtype=torch.float64, device=dev)
        for t in range(T):
            kt = K.kascade_topk_for_len(min(N, rule.tile * (t + 1)), rule)
            lst = ix[0, t, :, :kt].to(torch.int64).contiguous()        # [Hkv, kt]
            c = torch.searchsorted(lst, rows[t].expand(n_kv, -1).contiguous(), right=True)
            cnt += c.sum(dim=1).double()
        per_anchor[a] = cnt.cpu().numpy()
    total = 0.0
    for l in layers_reuse:
        c = per_anchor[anchor_of[l]]
        total += sum(c[int(maps[l][g])] for g in range(n_kv)) * group
    return 4.0 * d * total


def build_prefill(torch, K, synth, configs, dtype="bf16"):
    cfg = dataclasses.replace(configs.LLAMA_PREFILL_32K, dtype=dtype)
    N, L = cfg.ctx_len, cfg.n_layers
    lin = synth.heavy_lineages(cfg.seed, L, cfg.n_kv_heads, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, L, cfg.anchors, cfg.n_kv_heads, cfg.head_map_kind)
    layers = []
    for l in range(L):
        layers.append(synth.prefill_layer(cfg.seed, l, 1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, N,
                                          synth.layer_heavy_sets(lin, l, cfg.anchors, maps),
                                          cfg.alpha, cfg.gamma, cfg.dtype, device="cuda"))
    rule = K.PREFILL_RULE
    sh = K.make_shape(layers[0][0], layers[0][1], N)
    ws = K.workspace(K.OP_ANCHOR_PREFILL, sh, 0, rule)
    T = N // rule.tile
    kmax = K.kascade_topk_for_len(N, rule)
    idx = {a: torch.empty((1, T, cfg.n_kv_heads, kmax), dtype=torch.int32, device="cuda")
           for a in cfg.anchors}
    out = torch.empty_like(layers[0][0])
    anchor_of = {l: max(a for a in cfg.anchors if a <= l) for l in range(L)}

    lse = torch.empty(layers[0][0].shape[:3], dtype=torch.float32, device="cuda")

    def run(kind=None):
        if kind == "dense":   # the GPU's own dense causal prefill (comparison), one layer
            q, k, v = layers[0]
            K.check(K.kascade_dense_prefill(sh, q, k, v, out, lse), "dense_prefill")
            return
        for l, (q, k, v) in enumerate(layers):
            if l in cfg.anchors:
                if kind in (None, "anchor"):
                    K.check(K.kascade_anchor_prefill(sh, q, k, v, rule, out, None, idx[l], None, ws,
                                                     ws.numel()), "anchor_prefill")
            elif kind in (None, "reuse"):
                K.check(K.kascade_reuse_prefill(sh, q, k, v, rule, idx[anchor_of[l]], maps[l], out,
                                                None, 0), "reuse_prefill")

    d = cfg.head_dim
    flops_flash, flops_pool = prefill_flops(cfg)
    reuse_layers = [l for l in range(L) if l not in cfg.anchors]

    def reuse_flops():
        return prefill_reuse_flops(torch, K, idx, anchor_of, maps, reuse_layers, N, cfg.n_kv_heads,
                                   cfg.group, d)

    return dict(cfg=cfg, run=run, n_anchor=len(cfg.anchors), n_reuse=L - len(cfg.anchors),
                flops_flash=flops_flash, flops_pool=flops_pool, reuse_flops=reuse_flops,
                layers=layers, maps=maps)


def build_qwen3(torch, K, synth, configs, dtype="bf16"):
    """The Qwen3-8B-shaped end-to-end workload: 36 layers (32 query / 8 KV
    heads, d 128), 6 anchors chosen by the library's DP on the seeded
    similarity matrix, many-to-one head maps; a 65536-token causal prefill
    through every layer, then 512 generated tokens whose K/V rows sit in
    caches of 66048 rows (decode step s sees the first 65537 + s rows; its
    row was written at set-up, which leaves every step's inputs as if it had
    been appended)."""
    cfg = dataclasses.replace(configs.QWEN3_E2E_64K, dtype=dtype)
    L, Hq, Hkv, d, G = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.group
    N0, steps = cfg.ctx_len, cfg.decode_steps
    n_max = N0 + steps
    S = synth.similarity_matrix(cfg.seed, L)
    anchors, _ = K.kascade_select_anchors(L, cfg.n_anchor_dp, S)
    maps = synth.head_maps(cfg.seed, L, anchors, Hkv, cfg.head_map_kind)
    lin = synth.heavy_lineages(cfg.seed, L, Hkv, N0, cfg.heavy, cfg.drift)
    anchor_of = {l: max(a for a in anchors if a <= l) for l in range(L)}
    layers, qs = [], [[None] * L for _ in range(steps)]
    for l in range(L):
        q, k, v = synth.prefill_layer(cfg.seed, l, 1, Hq, Hkv, d, N0,
                                      synth.layer_heavy_sets(lin, l, anchors, maps),
                                      cfg.alpha, cfg.gamma, cfg.dtype, device="cuda", n_max=n_max)
        u = synth.prefill_directions(cfg.seed, l, Hkv, d, device="cuda")
        for st in range(steps):
            qd, kr, vr = synth.decode_step(cfg.seed, l, st, 1, Hq, Hkv, d, u, cfg.gamma, cfg.dtype,
                                           device="cuda")
            k[:, :, N0 + st] = kr
            v[:, :, N0 + st] = vr
            qs[st][l] = qd
        layers.append((q, k, v))
    rule = K.PREFILL_RULE
    sh = K.make_shape(layers[0][0], layers[0][1], N0)
    ws_p = K.workspace(K.OP_ANCHOR_PREFILL, sh, 0, rule)
    T = N0 // rule.tile
    kmax = K.kascade_topk_for_len(N0, rule)
    tidx = {a: torch.empty((1, T, Hkv, kmax), dtype=torch.int32, device="cuda") for a in anchors}
    out_p = torch.empty_like(layers[0][0])

    def prefill(kind=None):
        for l, (q, k, v) in enumerate(layers):
            if l in anchors:
                if kind in (None, "anchor"):
                    K.check(K.kascade_anchor_prefill(sh, q, k, v, rule, out_p, None, tidx[l], None, ws_p,
                                                     ws_p.numel()), "anchor_prefill")
            elif kind in (None, "reuse"):
                K.check(K.kascade_reuse_prefill(sh, q, k, v, rule, tidx[anchor_of[l]], maps[l], out_p,
                                                None, 0), "reuse_prefill")

    dec_k = lambda n: K.kascade_topk_for_len(n, K.DECODE_RULE)
    k_last = dec_k(n_max)
    sh_max = K.make_shape(qs[0][0], layers[0][1], n_max)
    ws_a = K.workspace(K.OP_ANCHOR_DECODE, sh_max, k_last)
    ws_r = K.workspace(K.OP_REUSE_DECODE, sh_max, k_last)
    ws_f = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh_max, k_last)
    didx = {a: torch.empty((1, Hkv, k_last), dtype=torch.int32, device="cuda") for a in anchors}
    out_d = torch.empty_like(qs[0][0])
    a0 = anchors[0]
    st0 = K.kascade_anchor_decode_fused(sh_max, qs[steps - 1][a0], layers[a0][1], layers[a0][2], k_last, out_d,
                                        None, didx[a0], None, 0, ws_f, ws_f.numel())
    if st0 not in (K.KASCADE_OK, K.KASCADE_ERR_SHAPE):
        K.check(st0, "anchor_decode_fused")
    fused_ok = st0 == K.KASCADE_OK

    def decode(st, kind=None):
        n_cur = N0 + st + 1
        kk = dec_k(n_cur)
        fused = kind == "anchor_fused" or (kind in (None, "anchor") and FUSED_ANCHOR and fused_ok)
        for l, (_, k, v) in enumerate(layers):
            shd = K.make_shape(qs[st][l], k, n_cur)
            if l in anchors:
                if kind in (None, "anchor", "anchor_fused") and fused:
                    K.check(K.kascade_anchor_decode_fused(shd, qs[st][l], k, v, kk, out_d, None, didx[l], None,
                                                          0, ws_f, ws_f.numel()), "anchor_decode_fused")
                elif kind in (None, "anchor"):
                    K.check(K.kascade_anchor_decode(shd, qs[st][l], k, v, kk, out_d, None, didx[l], None,
                                                    ws_a, ws_a.numel()), "anchor_decode")
            elif kind in (None, "reuse"):
                K.check(K.kascade_reuse_decode(shd, qs[st][l], k, v, kk, didx[anchor_of[l]], maps[l],
                                               out_d, ws_r, ws_r.numel()), "reuse_decode")

    reuse_layers = [l for l in range(L) if l not in anchors]

    def reuse_flops():
        return prefill_reuse_flops(torch, K, tidx, anchor_of, maps, reuse_layers, N0, Hkv, G, d)

    return dict(cfg=cfg, anchors=anchors, S=S, prefill=prefill, decode=decode, steps=steps, N0=N0,
                n_anchor=len(anchors), n_reuse=L - len(anchors), reuse_flops=reuse_flops, dec_k=dec_k,
                fused_ok=fused_ok)


# ---------------------------------------------------------------------------
# CPU oracle baseline on bounded samples (decode, prefill, anchor DP)
# ---------------------------------------------------------------------------

def host_info():
    """Host CPU model, the CPUs this process may run on and the BLAS threads."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    return model, affinity, blas


def cpu_baseline(dec, pre, torch):
    """The oracle, as it stands, on bounded samples of the workloads.

    value: 32K decode us/layer from one anchor and one reuse layer (weighted
    by the layer counts).  Also: the 32K prefill on 16 sampled tiles of one
    KV head (tiles 0, 1, 20, the last and 12 seeded others) of one anchor and
    one reuse layer, extrapolated to every tile and KV head (labelled
    extrapolated), and the anchor DP over the 36-layer similarity matrix."""
    import oracle
    model, affinity, blas = host_info()
    cfg = dec["cfg"]
    a = cfg.anchors[0]
    r = a + 1
    qa, ka, va = (x.float().cpu().numpy() for x in dec["layers"][a])
    qr, kr, vr = (x.float().cpu().numpy() for x in dec["layers"][r])
    t0 = time.perf_counter()
    reps_a = 0
    while True:
        _, _, _, ridx = oracle.anchor_decode(qa, ka, va, cfg.topk)
        reps_a += 1
        if time.perf_counter() - t0 > 3.0:
            break
    t_anchor = (time.perf_counter() - t0) / reps_a
    t1 = time.perf_counter()
    reps_r = 0
    while True:
        oracle.reuse_decode(qr, kr, vr, ridx, dec["maps"][r])
        reps_r += 1
        if time.perf_counter() - t1 > 2.0:
            break
    t_reuse = (time.perf_counter() - t1) / reps_r
    L = cfg.n_layers
    per_layer = (dec["n_anchor"] * t_anchor + dec["n_reuse"] * t_reuse) / L
    line = {"value": per_layer * 1e6, "unit": "us/layer", "cores": int(min(blas, affinity)),
            "kind": "oracle",
            "sample": "32K-context decode: one anchor layer (%d reps) and one reuse layer (%d reps), "
                      "weighted %d anchor : %d reuse layers" % (reps_a, reps_r, dec["n_anchor"],
                                                                 dec["n_reuse"]),
            "cpu_model": model, "affinity_cpus": affinity, "blas_threads": blas,
            "anchor_s": t_anchor, "reuse_s": t_reuse}
    if pre is not None:
        line["prefill32k"] = cpu_prefill_sample(pre, oracle)
    S = pre["qwen3_S"] if pre is not None and "qwen3_S" in pre else None
    if S is not None:
        t2 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t2 < 0.5:
            oracle.dp_select_anchors(S, 6)
            reps += 1
        line["anchor_dp_ms"] = (time.perf_counter() - t2) / reps * 1e3
        line["anchor_dp_sample"] = "36-layer seeded similarity matrix, 6 anchors (%d reps)" % reps
    return line


def cpu_prefill_sample(pre, oracle):
    cfg = pre["cfg"]
    N, Hkv, G, tile = cfg.ctx_len, cfg.n_kv_heads, cfg.group, 128
    T = N // tile
    rng = np.random.default_rng(cfg.seed)
    tiles = sorted(set([0, 1, 20, T - 1]) | set(int(x) for x in rng.choice(np.arange(2, T - 1), 12,
                                                                            replace=False)))
    a, r = cfg.anchors[0], cfg.anchors[0] + 1
    g = 0
    f64 = lambda t: t.float().cpu().numpy()
    qa, ka, va = (f64(x[:, g * G:(g + 1) * G] if i == 0 else x[:, g:g + 1])
                  for i, x in enumerate(pre["layers"][a]))
    qr, kr, vr = (f64(x[:, g * G:(g + 1) * G] if i == 0 else x[:, g:g + 1])
                  for i, x in enumerate(pre["layers"][r]))
    lists = {}
    t0 = time.perf_counter()
    for t in tiles:
        rows = range(tile * t, tile * (t + 1))
        for hh in range(G):
            oracle.dense_prefill_rows(qa, ka, va, 0, hh, rows)
        pooled = oracle.tile_pool_one(qa, ka, 0, t, 0)
        P, kt = oracle.prefill_tile_k(t, N)
        lists[t] = oracle.topk_full_sort(pooled, kt)
    t_anchor = time.perf_counter() - t0
    kmax = oracle.prefill_tile_k(T - 1, N)[1]
    idx = -np.ones((1, T, 1, kmax), dtype=np.int64)
    for t in tiles:
        idx[0, t, 0, :len(lists[t])] = lists[t]
    t1 = time.perf_counter()
    for t in tiles:
        rows = range(tile * t, tile * (t + 1))
        for hh in range(G):
            oracle.sparse_prefill_rows(qr, kr, vr, idx, [0], 0, hh, rows)
    t_reuse = time.perf_counter() - t1
    scale = T * Hkv / len(tiles)
    L = cfg.n_layers
    na = len(cfg.anchors)
    ms = (na * t_anchor * scale + (L - na) * t_reuse * scale) * 1e3
    return {"value": ms, "unit": "ms (32 layers, extrapolated)", "kind": "oracle",
            "extrapolated": True,
            "sample": "%d tiles (%s) of KV head 0 of one anchor and one reuse layer, x %d tiles x %d "
                      "KV heads / %d sampled" % (len(tiles), ",".join(map(str, tiles)), T, Hkv,
                                                 len(tiles)),
            "anchor_layer_s": t_anchor * scale, "reuse_layer_s": t_reuse * scale}


# ---------------------------------------------------------------------------
# HBM traffic (counter) support
# ---------------------------------------------------------------------------

def kernel_source_hash(kernel):
    """sha256 over the sources a kernel is built from (its .hip and the shared headers)."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "common.h", "kernels.h", "paged.h", "radix.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, config):
    """HBM bytes per launch of `kernel` on `config` from the stored counter summary.

    The summary holds lines `traffic | <kernel> | <config> | <bytes> | <source hash>`;
    the figure is returned only while the kernel's sources still hash the same,
    else None (the counters describe code that no longer exists)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    cur = kernel_source_hash(kernel)
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            parts = [x.strip() for x in line.strip().strip("|").split("|")]
            if len(parts) == 5 and parts[0] == "traffic" and parts[1] == kernel and parts[2] == config:
                return float(parts[3]) if parts[4] == cur else None
    return None


def traffic_probe(torch, K, synth, configs):
    """One launch of every kernel of the hot path, plus a plain copy of known size.

    Meant to run under `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE): the copy
    (an elementwise multiply by one reading and writing COPY_BYTES) calibrates
    the counters, which are then read per dispatch for each kernel."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1, out=dst)
    torch.cuda.synchronize()
    log("copy done")
    # prefill: one anchor layer and one reuse layer of the 32K prompt
    cfg = configs.LLAMA_PREFILL_32K
    N = cfg.ctx_len
    lin = synth.heavy_lineages(cfg.seed, cfg.n_layers, cfg.n_kv_heads, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, cfg.n_layers, cfg.anchors, cfg.n_kv_heads, cfg.head_map_kind)
    lay = [synth.prefill_layer(cfg.seed, l, 1, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, N,
                               synth.layer_heavy_sets(lin, l, cfg.anchors, maps), cfg.alpha,
                               cfg.gamma, cfg.dtype, device="cuda") for l in (0, 1)]
    rule = K.PREFILL_RULE
    sh = K.make_shape(lay[0][0], lay[0][1], N)
    ws = K.workspace(K.OP_ANCHOR_PREFILL, sh, 0, rule)
    T = N // rule.tile
    kmax = K.kascade_topk_for_len(N, rule)
    idx = torch.empty((1, T, cfg.n_kv_heads, kmax), dtype=torch.int32, device="cuda")
    out = torch.empty_like(lay[0][0])
    K.check(K.kascade_anchor_prefill(sh, *lay[0], rule, out, None, idx, None, ws, ws.numel()),
            "anchor_prefill")
    K.check(K.kascade_reuse_prefill(sh, *lay[1], rule, idx, maps[1], out, None, 0), "reuse_prefill")
    torch.cuda.synchronize()
    del lay, out, ws, idx
    log("prefill done")
    # decode: one anchor and one reuse layer at 128K context, batch 4
    cfg = configs.LLAMA_DECODE_128K
    N = cfg.ctx_len
    lin = synth.heavy_lineages(cfg.seed, cfg.n_layers, cfg.n_kv_heads, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, cfg.n_layers, cfg.anchors, cfg.n_kv_heads, cfg.head_map_kind)
    lay = [synth.decode_layer(cfg.seed, l, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, N,
                              synth.layer_heavy_sets(lin, l, cfg.anchors, maps), cfg.alpha, cfg.dtype,
                              device="cuda") for l in (0, 1)]
    sh = K.make_shape(lay[0][0], lay[0][1], N)
    ws_a = K.workspace(K.OP_ANCHOR_DECODE, sh, cfg.topk)
    ws_r = K.workspace(K.OP_REUSE_DECODE, sh, cfg.topk)
    idx = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(lay[0][0])
    K.check(K.kascade_anchor_decode(sh, *lay[0], cfg.topk, out, None, idx, None, ws_a, ws_a.numel()),
            "anchor_decode")
    K.check(K.kascade_reuse_decode(sh, *lay[1], cfg.topk, idx, maps[1], out, ws_r, ws_r.numel()),
            "reuse_decode")
    torch.cuda.synchronize()
    del lay, out, ws_a, ws_r, idx
    log("decode done")
    # the one-launch anchor decode: one layer at 32K context, batch 1
    cfg = configs.LLAMA_DECODE_32K
    N = cfg.ctx_len
    lin = synth.heavy_lineages(cfg.seed, cfg.n_layers, cfg.n_kv_heads, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, cfg.n_layers, cfg.anchors, cfg.n_kv_heads, cfg.head_map_kind)
    lay = synth.decode_layer(cfg.seed, 0, cfg.batch, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, N,
                             synth.layer_heavy_sets(lin, 0, cfg.anchors, maps), cfg.alpha, cfg.dtype,
                             device="cuda")
    sh = K.make_shape(lay[0], lay[1], N)
    ws_f = K.workspace(K.OP_ANCHOR_DECODE_FUSED, sh, cfg.topk)
    idx = torch.empty((cfg.batch, cfg.n_kv_heads, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(lay[0])
    K.check(K.kascade_anchor_decode_fused(sh, *lay, cfg.topk, out, None, idx, None, 0, ws_f, ws_f.numel()),
            "anchor_decode_fused")
    torch.cuda.synchronize()
    log("fused decode done")
    print(json.dumps({"probe": "traffic", "copy_bytes": COPY_BYTES,
                      "hashes": {k: kernel_source_hash(k) for k in KERNEL_SOURCES}}), flush=True)


def calibration_bench(torch, K, synth, configs, args):
    """Offline calibration on the 32K-context Llama-shaped decode layers: the
    anchor decode pass of every layer over S calibration queries (pooled rows
    and Top-k lists), the per-KV-head similarity of every layer pair, the
    weighted similarity, the anchor DP and the head maps.  Prints one JSON
    line; the oracle's similarity of one layer pair is timed beside it."""
    import oracle
    cfg = configs.LLAMA_DECODE_32K
    L, Hkv, N, k, S = cfg.n_layers, cfg.n_kv_heads, cfg.ctx_len, cfg.topk, 4
    lin = synth.heavy_lineages(cfg.seed, L, Hkv, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, L, cfg.anchors, Hkv, cfg.head_map_kind)
    pooled = torch.empty((L, S, Hkv, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((L, S, Hkv, k), dtype=torch.int32, device="cuda")
    layers = []
    for l in range(L):
        layers.append(synth.decode_layer(cfg.seed, l, S, cfg.n_q_heads, Hkv, cfg.head_dim, N,
                                         synth.layer_heavy_sets(lin, l, cfg.anchors, maps),
                                         cfg.alpha, cfg.dtype, device="cuda"))
    sh = K.make_shape(layers[0][0], layers[0][1], N)
    ws = K.workspace(K.OP_ANCHOR_DECODE, sh, k)
    out = torch.empty_like(layers[0][0])

    def passes():
        for l, (q, kk, v) in enumerate(layers):
            K.check(K.kascade_anchor_decode(sh, q, kk, v, k, out, None, idx[l], pooled[l], ws, ws.numel()),
                    "anchor_decode")

    sim = torch.zeros((L, L, Hkv, Hkv), dtype=torch.float32, device="cuda")

    def simk():
        K.check(K.kascade_calib_head_similarity(L, S, Hkv, N, k, pooled, idx, sim), "calib")

    for _ in range(args.warmup):
        passes()
        simk()
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    for _ in range(args.steps):
        passes()
    e[1].record()
    for _ in range(args.steps):
        simk()
    e[2].record()
    torch.cuda.synchronize()
    t_pass = e[0].elapsed_time(e[1]) / args.steps
    t_sim = e[1].elapsed_time(e[2]) / args.steps
    t0 = time.perf_counter()
    simh = sim.cpu().numpy()
    Sm = K.kascade_weighted_similarity(L, Hkv, simh, None)
    anchors, _ = K.kascade_select_anchors(L, len(cfg.anchors), Sm)
    K.kascade_head_maps(L, Hkv, simh, anchors)
    t_host = (time.perf_counter() - t0) * 1e3
    pairs = L * (L + 1) // 2
    gathered = pairs * Hkv * S * (Hkv + 1) * k * 4
    # oracle on one layer pair (S queries), the same quantity
    rp = []
    for l in (0, 1):
        q, kk, v = layers[l]
        rp.append(oracle.anchor_decode(*(x.float().cpu().numpy().astype(np.float64) for x in (q, kk, v)), k)[2])
    t1 = time.perf_counter()
    oracle.head_similarity(rp[0], rp[1], k)
    t_oracle_pair = time.perf_counter() - t1
    print(json.dumps({
        "metric": "calibration: per-KV-head similarity of all layer pairs (ms)", "value": t_sim,
        "unit": "ms", "higher_is_better": False, "dtype": "f32 pooled rows, f64 sums",
        "config": {"workload": "Llama-3.1-8B-shaped decode layers, 32 layers, 8 KV heads, 32K ctx, "
                               "k=3264, %d calibration queries" % S},
        "anchor_passes_ms": t_pass, "similarity_ms": t_sim, "host_dp_headmaps_ms": t_host,
        "layer_pairs": pairs, "gathered_GBps": gathered / (t_sim * 1e-3) / 1e9,
        "anchors": anchors,
        "cpu_baseline": {"value": t_oracle_pair * pairs * 1e3, "unit": "ms", "kind": "oracle",
                         "sample": "one layer pair timed (%.2f s), x %d pairs" % (t_oracle_pair, pairs)},
    }), flush=True)


def paged_bench(torch, K, synth, configs, args):
    """Decode over paged caches (block size 16, blocks scattered by a seeded
    permutation) against the same layers in contiguous caches, on the 32K
    (B=1) and 128K (B=4) Llama-shaped workloads with 8 distinct layers each.
    Prints one JSON line."""
    res = {}
    for cfg, name in ((configs.LLAMA_DECODE_32K, "decode32k"), (configs.LLAMA_DECODE_128K, "decode128k")):
        N, B, Hkv, k = cfg.ctx_len, cfg.batch, cfg.n_kv_heads, cfg.topk
        bs, nl = 16, 8
        lin = synth.heavy_lineages(cfg.seed, nl, Hkv, N, cfg.heavy, cfg.drift)
        maps = synth.head_maps(cfg.seed, nl, (0,), Hkv, cfg.head_map_kind)
        nb = N // bs
        rng = np.random.default_rng(cfg.seed)
        layers = []
        for l in range(nl):
            q, kk, v = synth.decode_layer(cfg.seed, l, B, cfg.n_q_heads, Hkv, cfg.head_dim, N,
                                          synth.layer_heavy_sets(lin, l, (0,), maps), cfg.alpha, cfg.dtype,
                                          device="cuda")
            perm = torch.as_tensor(rng.permutation(B * nb).reshape(B, nb), dtype=torch.int64, device="cuda")
            kc = torch.empty((B * nb, Hkv, bs, cfg.head_dim), dtype=kk.dtype, device="cuda")
            vc = torch.empty_like(kc)
            kc[perm.reshape(-1)] = kk.view(B, Hkv, nb, bs, -1).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, -1)
            vc[perm.reshape(-1)] = v.view(B, Hkv, nb, bs, -1).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, -1)
            layers.append((q, kk, v, kc, vc, perm.to(torch.int32).contiguous()))
        sh = K.make_shape(layers[0][0], layers[0][1], N)
        shp = K.paged_shape(layers[0][0], layers[0][3], N)
        ws_a = K.workspace(K.OP_ANCHOR_DECODE, sh, k)
        ws_r = K.workspace(K.OP_REUSE_DECODE, sh, k)
        idx = torch.empty((B, Hkv, k), dtype=torch.int32, device="cuda")
        out = torch.empty_like(layers[0][0])

        def run(kind, paged):
            for q, kk, v, kc, vc, tab in layers:
                if paged:
                    pg = K.paged_kv(tab, kc)
                    if kind == "anchor":
                        K.check(K.kascade_anchor_decode_paged(shp, pg, q, kc, vc, k, out, None, idx, None, ws_a,
                                                              ws_a.numel()), "anchor_paged")
                    else:
                        K.check(K.kascade_reuse_decode_paged(shp, pg, q, kc, vc, k, idx, maps[1], out, ws_r,
                                                             ws_r.numel()), "reuse_paged")
                elif kind == "anchor":
                    K.check(K.kascade_anchor_decode(sh, q, kk, v, k, out, None, idx, None, ws_a, ws_a.numel()),
                            "anchor")
                else:
                    K.check(K.kascade_reuse_decode(sh, q, kk, v, k, idx, maps[1], out, ws_r, ws_r.numel()),
                            "reuse")

        row = {}
        for kind in ("anchor", "reuse"):
            for paged in (False, True):
                # the kind's 8 layers as one HIP graph, timed over primed replays
                g = capture_graph(torch, lambda kind=kind, paged=paged: run(kind, paged))
                for _ in range(args.warmup):
                    g.replay()
                us = float(np.median(event_reps(torch, g.replay, max(args.steps, 10)))) * 1e3 / nl
                del g
                by = 2 * B * Hkv * (N if kind == "anchor" else k) * cfg.head_dim * 2
                row["%s_%s_us" % (kind, "paged" if paged else "contig")] = us
                row["%s_%s_GBps" % (kind, "paged" if paged else "contig")] = by / (us * 1e-6) / 1e9
        res[name] = row
        del layers
        torch.cuda.empty_cache()
    res["prefill32k"] = paged_prefill_row(torch, K, synth, configs, args)
    print(json.dumps({"metric": "paged-KV attention (block size 16) vs contiguous: decode us/layer, "
                                "reuse prefill ms/layer",
                      "unit": "us/layer", "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "Llama-3.1-8B-shaped layers, 32q/8kv heads, d=128: decode "
                                             "32K B=1 k=3264 and 128K B=4 k=13120 (8 distinct layers), "
                                             "reuse prefill of a 32K-token prompt (tile 128, k_t min 256)"},
                      "components": res}), flush=True)


def paged_prefill_row(torch, K, synth, configs, args):
    """Reuse prefill of the 32K-token prompt over a paged cache (block size
    16, blocks scattered by a seeded permutation) against the contiguous
    cache, on the tile lists of the anchor layer before it; the two outputs
    must be bitwise identical."""
    cfg = configs.LLAMA_PREFILL_32K
    N, Hkv, d, bs = cfg.ctx_len, cfg.n_kv_heads, cfg.head_dim, 16
    lin = synth.heavy_lineages(cfg.seed, 2, Hkv, N, cfg.heavy, cfg.drift)
    maps = synth.head_maps(cfg.seed, 2, (0,), Hkv, cfg.head_map_kind)
    lay = [synth.prefill_layer(cfg.seed, l, 1, cfg.n_q_heads, Hkv, d, N, synth.layer_heavy_sets(lin, l, (0,), maps),
                               cfg.alpha, cfg.gamma, cfg.dtype, device="cuda") for l in (0, 1)]
    _, _, tidx, _ = K.anchor_prefill(*lay[0])
    q, kk, v = lay[1]
    nb = N // bs
    perm = torch.as_tensor(np.random.default_rng(cfg.seed).permutation(nb), dtype=torch.int64, device="cuda")
    kc = torch.empty((nb, Hkv, bs, d), dtype=kk.dtype, device="cuda")
    vc = torch.empty_like(kc)
    kc[perm] = kk.view(Hkv, nb, bs, d).permute(1, 0, 2, 3)
    vc[perm] = v.view(Hkv, nb, bs, d).permute(1, 0, 2, 3)
    tab = perm.to(torch.int32).view(1, nb).contiguous()
    sh = K.make_shape(q, kk, N)
    shp = K.paged_shape(q, kc, N)
    pg = K.paged_kv(tab, kc)
    outs = {False: torch.empty_like(q), True: torch.empty_like(q)}

    def run(paged):
        if paged:
            K.check(K.kascade_reuse_prefill_paged(shp, pg, q, kc, vc, K.PREFILL_RULE, tidx, maps[1], outs[True]),
                    "reuse_prefill_paged")
        else:
            K.check(K.kascade_reuse_prefill(sh, q, kk, v, K.PREFILL_RULE, tidx, maps[1], outs[False], None, 0),
                    "reuse_prefill")

    row = {}
    for paged in (False, True):
        for _ in range(args.warmup):
            run(paged)
        torch.cuda.synchronize()
        ts = event_reps(torch, lambda: run(paged), max(args.steps, 5), prime=False)
        row["reuse_%s_ms" % ("paged" if paged else "contig")] = float(np.median(ts))
    row["identical"] = bool(torch.equal(outs[False].view(torch.int16), outs[True].view(torch.int16)))
    return row


# ---------------------------------------------------------------------------

def capture_graph(torch, fn):
    """fn() (library calls on torch's current stream) captured as one HIP graph.
    One eager run on the capture stream comes first, so the library's
    once-per-device set-up happens outside the capture."""
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fn()
        with torch.cuda.graph(g, stream=st):
            fn()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    return g


def event_reps(torch, fn, reps, prime=True):
    """Milliseconds of each of `reps` runs of fn(), each bracketed by HIP events
    on the current stream and followed by a synchronisation.  prime: one
    untimed fn() is queued first, so the timed call is submitted while the GPU
    is busy and the window holds its execution, not the ~30 us it takes to
    hand a HIP graph (or the first kernel) to an idle GPU."""
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if prime:
            fn()
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return np.asarray(ts)


def pct(ts, scale=1.0):
    """median, p10 and p90 of a sample, times `scale`."""
    return {"median": float(np.median(ts)) * scale, "p10": float(np.percentile(ts, 10)) * scale,
            "p90": float(np.percentile(ts, 90)) * scale, "n": int(len(ts))}


def stream_copy_gbps(torch, nbytes=4 << 30, reps=10):
    """Measured HBM copy bandwidth (bytes read + written per second) of torch's
    device copy over a buffer far larger than the last-level cache."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = event_reps(torch, lambda: dst.copy_(src), reps)
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * nbytes / (np.median(ts) * 1e-3) / 1e9


def stream_read_gbps(torch, K, nbytes=4 << 30, reps=10):
    """Measured HBM read bandwidth: the library's stream-read reference
    (kascade_stream_read: every byte read once with the decode passes'
    16-byte nontemporal loads) over a buffer far larger than the last-level
    cache."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    run = lambda: K.check(K.kascade_stream_read(src, nbytes, sink), "kascade_stream_read")
    run()
    ts = event_reps(torch, run, reps)
    del src, sink
    torch.cuda.empty_cache()
    return nbytes / (np.median(ts) * 1e-3) / 1e9


def qwen3_bench(torch, K, synth, configs, args, reps):
    """Config-5 figures: the 36-layer 64K prefill (eager; per kind over the
    layers of that kind) and the 512 decode steps, each step one HIP graph,
    replayed back to back; per-kind decode figures from graphs of the last
    step's anchor or reuse layers."""
    w = build_qwen3(torch, K, synth, configs, args.dtype)
    cfg = w["cfg"]
    L, Hq, Hkv, d = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    N0, steps = w["N0"], w["steps"]
    na, nr = w["n_anchor"], w["n_reuse"]
    log("qwen3: anchors", w["anchors"])
    w["prefill"]()
    torch.cuda.synchronize()
    pre = {}
    for kind in (None, "anchor", "reuse"):
        pre[kind] = event_reps(torch, lambda: w["prefill"](kind), 3, prime=False)
    rf = w["reuse_flops"]()
    fl_anchor = sum(prefill_flops(cfg))
    anchor_ms = float(np.median(pre["anchor"])) / na
    reuse_ms = float(np.median(pre["reuse"])) / nr
    log("qwen3: prefill done, capturing %d decode steps" % steps)
    graphs = [capture_graph(torch, lambda st=st: w["decode"](st)) for st in range(steps)]
    for g in graphs[:8]:
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    passes = []
    per_step = []
    for _ in range(3):
        ev[0].record()
        for st, g in enumerate(graphs):
            g.replay()
            ev[st + 1].record()
        torch.cuda.synchronize()
        passes.append(ev[0].elapsed_time(ev[steps]))
        per_step += [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    del graphs
    last = steps - 1
    n_last = N0 + steps
    kind_us = {}
    kinds = (("anchor", na), ("reuse", nr)) + ((("anchor_fused", na),) if w["fused_ok"] else ())
    for kind, n in kinds:
        g = capture_graph(torch, lambda kind=kind: w["decode"](last, kind))
        kind_us[kind] = pct(event_reps(torch, g.replay, reps), 1e3 / n)
        del g
    k_last = w["dec_k"](n_last)
    by_anchor, by_reuse, _ = decode_bytes(dataclasses.replace(cfg, ctx_len=n_last, topk=k_last, batch=1))
    torch.cuda.synchronize()
    res = {
        "workload": "Qwen3-8B-shaped: 36 layers, 32q/8kv heads, d=128, %s; DP anchors %s; prefill %d tokens "
                    "(tile 128, k_t min 256), then %d decode steps (k %d -> %d)" % (
                        args.dtype, w["anchors"], N0, steps, w["dec_k"](N0 + 1), k_last),
        "prefill_ms": float(np.median(pre[None])), "prefill_ms_runs": [float(x) for x in pre[None]],
        "prefill_anchor_ms_per_layer": anchor_ms, "prefill_reuse_ms_per_layer": reuse_ms,
        "prefill_anchor_TFLOPs": fl_anchor / (anchor_ms * 1e-3) / 1e12,
        "prefill_anchor_mfma_frac": fl_anchor / (anchor_ms * 1e-3) / 1e12 / MFMA16_PEAK_TFLOPS,
        "prefill_anchor_ideal_ms": fl_anchor / (MFMA16_PEAK_TFLOPS * 1e12) * 1e3,
        "prefill_reuse_TFLOPs": rf / nr / (reuse_ms * 1e-3) / 1e12,
        "prefill_reuse_mfma_frac": rf / nr / (reuse_ms * 1e-3) / 1e12 / MFMA16_PEAK_TFLOPS,
        "prefill_reuse_ideal_ms": rf / nr / (MFMA16_PEAK_TFLOPS * 1e12) * 1e3,
        "decode_ms_512_steps": float(np.median(passes)),
        "decode_us_per_layer": pct(np.asarray(per_step), 1e3 / L),
        "decode_anchor_us_last_step": kind_us["anchor"], "decode_reuse_us_last_step": kind_us["reuse"],
        "decode_anchor_fused_us_last_step": kind_us.get("anchor_fused"),
        "anchor_decode_path": "fused" if FUSED_ANCHOR and w["fused_ok"] else "split",
        "decode_anchor_ideal_us": by_anchor / (HBM_PEAK_GBS * 1e9) * 1e6,
        "decode_reuse_ideal_us": by_reuse / (HBM_PEAK_GBS * 1e9) * 1e6,
        "decode_anchor_hbm_frac": by_anchor / (kind_us["anchor"]["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "decode_reuse_hbm_frac": by_reuse / (kind_us["reuse"]["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
    }
    S = w["S"]
    del w
    torch.cuda.empty_cache()
    return res, S


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--reps", type=int, default=50,
                    help="repetitions of each section and kind for the median/p10/p90 figures")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qwen3", action="store_true",
                    help="skip the Qwen3-shaped 64K prefill + 512-step decode component")
    ap.add_argument("--only", choices=["decode32k", "decode128k", "prefill", "qwen3"], default=None,
                    help="run one section only (profiling)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the decode sections eagerly instead of replaying HIP graphs")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="one launch of each kernel plus a calibration copy, for rocprofv3 --pmc")
    ap.add_argument("--calibration", action="store_true",
                    help="time the offline calibration path (layer-pair similarities, DP, head maps)")
    ap.add_argument("--dtype", choices=["bf16", "f16"], default="bf16",
                    help="element type of q, k, v and outputs (the workloads are defined in bf16)")
    ap.add_argument("--paged", action="store_true",
                    help="time decode and the reuse prefill over paged KV caches against contiguous caches")
    ap.add_argument("--anchor-decode", choices=["split", "fused"], default="split",
                    help="anchor decode layers of the timed sections: four launches (split) or the "
                         "one-launch kernel where it fits (fused); both are timed per kind either way")
    args = ap.parse_args()
    global FUSED_ANCHOR
    FUSED_ANCHOR = args.anchor_decode == "fused"
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_anchor_amd import configs, synth
    from long_context_anchor_amd import kascade as K

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    K.lib()  # fails loudly when the HIP library is missing
    torch.cuda.set_device(0)
    if args.traffic_probe:
        traffic_probe(torch, K, synth, configs)
        return
    if args.calibration:
        calibration_bench(torch, K, synth, configs, args)
        return
    if args.paged:
        paged_bench(torch, K, synth, configs, args)
        return
    reps = max(args.reps, 1)
    if args.only == "qwen3":
        res, _ = qwen3_bench(torch, K, synth, configs, args, reps)
        print(json.dumps({"metric": METRIC, "config": {"workload": res["workload"]}, "qwen3_e2e": res}),
              flush=True)
        return

    # the 128K section goes first: the 32K graph is then handed over while the
    # GPU is busy, so its window holds execution only (the first section of a
    # step also holds the ~30 us hand-over of its graph to the idle GPU)
    sections = ["decode128k", "decode32k", "prefill"] if args.only is None else [args.only]
    log("building workloads", sections)
    t_build = time.perf_counter()
    work = {}
    if "decode32k" in sections or not args.no_cpu_baseline:
        work["decode32k"] = build_decode(configs.LLAMA_DECODE_32K, torch, K, synth, configs, args.dtype)
    if "decode128k" in sections:
        work["decode128k"] = build_decode(configs.LLAMA_DECODE_128K, torch, K, synth, configs, args.dtype)
    if "prefill" in sections or not args.no_cpu_baseline:
        work["prefill"] = build_prefill(torch, K, synth, configs, args.dtype)
    torch.cuda.synchronize()
    log("built in %.1f s" % (time.perf_counter() - t_build))

    # decode sections run as HIP graphs of their 32 layers (one per kind as
    # well), so their time is the GPU's and not the host's launch rate
    graphs = {}
    for s in ("decode32k", "decode128k"):
        if s in sections:
            w = work[s]
            kinds = (None, "anchor", "reuse", "dense") + (("anchor_fused",) if w["fused_ok"] else ())
            if args.eager:
                graphs[s] = {kind: (lambda kind=kind, w=w: w["run"](kind)) for kind in kinds}
            else:
                graphs[s] = {kind: capture_graph(torch, lambda kind=kind, w=w: w["run"](kind)).replay
                             for kind in kinds}
    log("decode graphs captured" if not args.eager else "eager decode")

    def run_section(s):
        if s == "prefill":
            work["prefill"]["run"]()
        else:
            graphs[s][None]()

    def step():
        marks = {}
        for s in sections:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            run_section(s)
            e1.record()
            marks[s] = (e0, e1)
        torch.cuda.synchronize()   # step boundary
        return marks

    for i in range(args.warmup):
        step()
        log("warmup step %d done" % i)

    # pick the kernel with the largest share of one eager step, then time it
    # live with the library's events during the timed steps (prefill kernels
    # run eagerly there; a decode kernel is timed over eager passes after them)
    for kid in range(8):
        K.kascade_kernel_timer_enable(kid, True)
    for s in sections:
        work[s]["run"]()
    torch.cuda.synchronize()
    shares = {kid: K.kascade_kernel_timer_read(kid) for kid in range(8)}
    for kid in range(8):
        K.kascade_kernel_timer_enable(kid, False)
    dom = max(shares, key=lambda k: shares[k][0])
    log("kernel shares (ms, launches):", {k: (round(v[0], 3), v[1]) for k, v in shares.items()})
    K.kascade_kernel_timer_enable(dom, True)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all_marks = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if dom < 5 and not args.eager:
        dsec = "decode128k" if "decode128k" in sections else "decode32k"
        for _ in range(max(1, min(args.steps, 10))):
            work[dsec]["run"]()
        torch.cuda.synchronize()
    dom_ms, dom_n = K.kascade_kernel_timer_read(dom)
    K.kascade_kernel_timer_enable(dom, False)
    log("timed %d steps in %.3f s" % (args.steps, wall))

    sec_ms = {s: np.asarray([m[s][0].elapsed_time(m[s][1]) for m in all_marks]) for s in sections}

    comps = {}
    for s in ("decode32k", "decode128k"):
        if s not in sections:
            continue
        w = work[s]
        L = w["cfg"].n_layers
        by = w["n_anchor"] * w["bytes_anchor"] + w["n_reuse"] * w["bytes_reuse"]
        us_layer = float(np.median(sec_ms[s])) * 1e3 / L
        # each section and kind again, `reps` times, one synchronised replay each
        rep = {None: pct(event_reps(torch, graphs[s][None], reps), 1e3 / L)}
        for kind, n in (("anchor", w["n_anchor"]), ("reuse", w["n_reuse"]), ("dense", L),
                        ("anchor_fused", w["n_anchor"])):
            if kind in graphs[s]:
                rep[kind] = pct(event_reps(torch, graphs[s][kind], reps), 1e3 / n)
        per = {k: rep[k]["median"] for k in ("anchor", "reuse", "dense")}
        comps[s] = {
            "us_per_layer": us_layer,
            "us_per_layer_steps": pct(sec_ms[s], 1e3 / L),
            "us_per_layer_reps": rep[None],
            "GBps": by / (us_layer * L * 1e-6) / 1e9,
            "hbm_frac": by / (us_layer * L * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "anchor_us": per["anchor"], "reuse_us": per["reuse"],
            "anchor_us_reps": rep["anchor"], "reuse_us_reps": rep["reuse"],
            # the one-launch anchor decode, per anchor layer (null where its
            # workgroups do not all fit on the GPU at once)
            "anchor_fused_us": rep["anchor_fused"]["median"] if "anchor_fused" in rep else None,
            "anchor_fused_us_reps": rep.get("anchor_fused"),
            "anchor_decode_path": "fused" if FUSED_ANCHOR and w["fused_ok"] else "split",
            "anchor_GBps": w["bytes_anchor"] / (per["anchor"] * 1e-6) / 1e9,
            "reuse_GBps": w["bytes_reuse"] / (per["reuse"] * 1e-6) / 1e9,
            "reuse_hbm_frac": w["bytes_reuse"] / (per["reuse"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "dense_us_per_layer": per["dense"], "dense_us_reps": rep["dense"],
            "dense_GBps": w["bytes_dense"] / (per["dense"] * 1e-6) / 1e9,
            "speedup_vs_dense": per["dense"] / us_layer,
            "context": w["cfg"].ctx_len, "batch": w["cfg"].batch, "topk": w["cfg"].topk,
            "timing": "eager launches" if args.eager else "HIP graph replay of the section's layers",
        }
    if "prefill" in sections:
        w = work["prefill"]
        rf = w["reuse_flops"]()
        fl = w["n_anchor"] * (w["flops_flash"] + w["flops_pool"]) + rf
        prep = max(3, min(reps, 10))
        per = {}
        rep = {}
        for kind, n in (("anchor", w["n_anchor"]), ("reuse", w["n_reuse"]), ("dense", 1)):
            rep[kind] = pct(event_reps(torch, lambda kind=kind: w["run"](kind), prep, prime=False), 1.0 / n)
            per[kind] = rep[kind]["median"]
        ms = float(np.median(sec_ms["prefill"]))
        comps["prefill32k"] = {
            "ms": ms, "ms_steps": pct(sec_ms["prefill"]), "TFLOPs": fl / (ms * 1e-3) / 1e12,
            "anchor_ms": per["anchor"], "reuse_ms": per["reuse"],
            "anchor_ms_reps": rep["anchor"], "reuse_ms_reps": rep["reuse"],
            "anchor_TFLOPs": (w["flops_flash"] + w["flops_pool"]) / (per["anchor"] * 1e-3) / 1e12,
            "reuse_TFLOPs": rf / w["n_reuse"] / (per["reuse"] * 1e-3) / 1e12,
            "mfma_frac": fl / (ms * 1e-3) / 1e12 / MFMA16_PEAK_TFLOPS,
            "anchor_mfma_frac": (w["flops_flash"] + w["flops_pool"]) / (per["anchor"] * 1e-3) / 1e12
            / MFMA16_PEAK_TFLOPS,
            "reuse_mfma_frac": rf / w["n_reuse"] / (per["reuse"] * 1e-3) / 1e12 / MFMA16_PEAK_TFLOPS,
            "dense_ms_per_layer": per["dense"],
            "dense_TFLOPs": w["flops_flash"] / (per["dense"] * 1e-3) / 1e12,
            "speedup_vs_dense": per["dense"] * w["cfg"].n_layers / ms,
        }

    # roofline of the dominant kernel
    names = {0: "decode_splitk", 1: "decode_combine", 2: "decode_pool", 3: "topk_select",
             4: "reuse_decode", 5: "prefill_flash", 6: "prefill_pool", 7: "prefill_sparse"}
    avg_ms = dom_ms / max(dom_n, 1)
    roof = {"kernel": names[dom], "launches": dom_n, "avg_ms": avg_ms}
    if dom in (5, 6, 7) and "prefill" in sections:
        w = work["prefill"]
        if dom == 5:
            per_launch = w["flops_flash"]
        elif dom == 6:
            per_launch = w["flops_pool"]
        else:
            per_launch = w["reuse_flops"]() / w["n_reuse"]
        ach = per_launch / (avg_ms * 1e-3) / 1e12
        roof.update({"bound": "mfma", "achieved": ach, "peak": MFMA16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": ach / MFMA16_PEAK_TFLOPS, "algorithmic_per_launch": per_launch,
                     "traffic": stored_traffic(names[dom], "prefill32k")})
    else:
        # decode kernels: algorithmic bytes of the launch (cache K+V or gathered rows)
        s = "decode128k" if "decode128k" in sections else "decode32k"
        w = work[s]
        per_launch = w["bytes_reuse"] if dom == 4 else w["bytes_anchor"]
        ach = per_launch / (avg_ms * 1e-3) / 1e9
        roof.update({"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "algorithmic_per_launch": per_launch,
                     "traffic": stored_traffic(names[dom], s)})

    # the decode sections' bandwidth against a measured stream read (and a
    # device copy) as well
    read_gbps = stream_read_gbps(torch, K)
    copy_gbps = stream_copy_gbps(torch)
    for s in ("decode32k", "decode128k"):
        if s in comps:
            comps[s]["stream_read_GBps"] = read_gbps
            comps[s]["reuse_frac_of_read"] = comps[s]["reuse_GBps"] / read_gbps
            comps[s]["anchor_frac_of_read"] = comps[s]["anchor_GBps"] / read_gbps
            comps[s]["stream_copy_GBps"] = copy_gbps
            comps[s]["reuse_frac_of_copy"] = comps[s]["reuse_GBps"] / copy_gbps
            comps[s]["anchor_frac_of_copy"] = comps[s]["anchor_GBps"] / copy_gbps

    qwen3_S = None
    if args.only is None and not args.no_qwen3:
        for s in ("decode32k", "decode128k"):
            graphs.pop(s, None)
        for s in ("decode128k",):
            work.pop(s, None)
        torch.cuda.empty_cache()
        comps["qwen3_e2e"], qwen3_S = qwen3_bench(torch, K, synth, configs, args, reps)

    ms_per_step = wall * 1e3 / args.steps
    value = comps.get("decode32k", {}).get("us_per_layer")
    line = {
        "metric": METRIC, "value": value, "unit": "us/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped attention, 32 layers, 32q/8kv heads, d=128, "
                               "anchors [0,2,8,13,14]: decode 32K ctx B=1 k=3264 + decode 128K ctx "
                               "B=4 k=13120 + prefill 32K tokens (tile 128, k_t min 256)",
                   "sections": sections,
                   "value": "median over the timed steps of the 32K decode section (32 layers, one "
                            "HIP graph replay) per layer"},
        "components": comps, "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        pre = work.get("prefill")
        if pre is not None and qwen3_S is not None:
            pre["qwen3_S"] = qwen3_S
        line["cpu_baseline"] = cpu_baseline(work["decode32k"], pre, torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

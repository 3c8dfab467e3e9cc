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
MFMA16_PEAK_TFLOPS = 2500.0  # dense bf16 and fp16 MFMA peak
# HBM traffic of the kernels, read by rocprofv3 counters and stored as text
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_kernels_llama8b.md")
CSRC = os.path.join(ROOT, "long_context_anchor_amd", "csrc")
KERNEL_SOURCES = {"prefill_flash": "prefill.hip", "prefill_pool": "prefill.hip",
                  "prefill_sparse": "prefill.hip", "decode_splitk": "decode.hip",
                  "decode_combine": "decode.hip", "decode_pool": "decode.hip",
                  "reuse_decode": "decode.hip", "topk_select": "select.hip",
                  "topk_select_wide_a": "select.hip", "topk_select_wide_b": "select.hip",
                  "topk_select_wide_c": "select.hip"}
COPY_BYTES = 1 << 30  # the calibration copy reads and writes this many bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# workload construction (synthetic, seeded)
# ---------------------------------------------------------------------------

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

    def run(kind=None):
        if kind == "dense":   # the GPU's own dense decode on every layer (comparison)
            for q, k, v in layers:
                K.check(K.kascade_dense_decode(sh, q, k, v, out, lse, ws_d, ws_d.numel()), "dense_decode")
            return
        for l, (q, k, v) in enumerate(layers):
            if l in cfg.anchors:
                if kind in (None, "anchor"):
                    K.check(K.kascade_anchor_decode(sh, q, k, v, cfg.topk, out, None, idx[l], None,
                                                    ws_a, ws_a.numel()), "anchor_decode")
            elif kind in (None, "reuse"):
                K.check(K.kascade_reuse_decode(sh, q, k, v, cfg.topk, idx[anchor_of[l]], maps[l], out,
                                               ws_r, ws_r.numel()), "reuse_decode")

    e = 2
    n_anchor = len(cfg.anchors)
    n_reuse = L - n_anchor
    io = cfg.batch * cfg.n_q_heads * cfg.head_dim * e * 2 + cfg.batch * cfg.n_kv_heads * cfg.topk * 4
    bytes_anchor = 2 * cfg.batch * cfg.n_kv_heads * N * cfg.head_dim * e + io
    bytes_reuse = 2 * cfg.batch * cfg.n_kv_heads * cfg.topk * cfg.head_dim * e + io
    bytes_dense = 2 * cfg.batch * cfg.n_kv_heads * N * cfg.head_dim * e + \
        cfg.batch * cfg.n_q_heads * cfg.head_dim * e * 2
    return dict(cfg=cfg, run=run, n_anchor=n_anchor, n_reuse=n_reuse, bytes_anchor=bytes_anchor,
                bytes_reuse=bytes_reuse, bytes_dense=bytes_dense, layers=layers, maps=maps)


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

    d, Hq = cfg.head_dim, cfg.n_q_heads
    flops_flash = 4.0 * d * Hq * N * (N + 1) / 2
    flops_pool = 2.0 * d * Hq * N * (N + 1) / 2

    def reuse_flops():
        # 4*d*sum_{h,r} |J_{h,r}|, counted from the anchors' lists
        total = 0.0
        rows = torch.arange(N, device="cuda", dtype=torch.int64).view(T, rule.tile)
        per_anchor = {}
        for a, ix in idx.items():
            cnt = torch.zeros(cfg.n_kv_heads, dtype=torch.float64, device="cuda")
            for t in range(T):
                P = min(N, rule.tile * (t + 1))
                kt = K.kascade_topk_for_len(P, rule)
                lst = ix[0, t, :, :kt].to(torch.int64).contiguous()        # [Hkv, kt]
                c = torch.searchsorted(lst, rows[t].expand(cfg.n_kv_heads, -1).contiguous(), right=True)
                cnt += c.sum(dim=1).double()
            per_anchor[a] = cnt.cpu().numpy()
        for l in range(L):
            if l in cfg.anchors:
                continue
            c = per_anchor[anchor_of[l]]
            total += sum(c[int(maps[l][g])] for g in range(cfg.n_kv_heads)) * cfg.group
        return 4.0 * d * total

    return dict(cfg=cfg, run=run, n_anchor=len(cfg.anchors), n_reuse=L - len(cfg.anchors),
                flops_flash=flops_flash, flops_pool=flops_pool, reuse_flops=reuse_flops)


# ---------------------------------------------------------------------------
# CPU oracle baseline on a bounded sample of the 32K decode workload
# ---------------------------------------------------------------------------

def cpu_baseline(dec, torch):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
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
        if time.perf_counter() - t0 > 6.0:
            break
    t_anchor = (time.perf_counter() - t0) / reps_a
    t1 = time.perf_counter()
    reps_r = 0
    while True:
        oracle.reuse_decode(qr, kr, vr, ridx, dec["maps"][r])
        reps_r += 1
        if time.perf_counter() - t1 > 4.0:
            break
    t_reuse = (time.perf_counter() - t1) / reps_r
    L = cfg.n_layers
    per_layer = (dec["n_anchor"] * t_anchor + dec["n_reuse"] * t_reuse) / L
    return {"value": per_layer * 1e6, "unit": "us/layer", "cores": int(threads), "kind": "oracle",
            "sample": "32K-context decode: one anchor layer (%d reps) and one reuse layer (%d reps), "
                      "weighted %d anchor : %d reuse layers; host %s, %d logical cpus" % (
                          reps_a, reps_r, dec["n_anchor"], dec["n_reuse"], platform.processor() or
                          platform.machine(), os.cpu_count() or 0),
            "anchor_s": t_anchor, "reuse_s": t_reuse}


# ---------------------------------------------------------------------------
# HBM traffic (counter) support
# ---------------------------------------------------------------------------

def kernel_source_hash(kernel):
    """sha256 over the sources a kernel is built from (its .hip and the shared headers)."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "common.h", "kernels.h"):
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
    log("decode done")
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
                for _ in range(args.warmup):
                    run(kind, paged)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(args.steps):
                    run(kind, paged)
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (args.steps * nl)
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
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            run(paged)
        e1.record()
        torch.cuda.synchronize()
        row["reuse_%s_ms" % ("paged" if paged else "contig")] = e0.elapsed_time(e1) / args.steps
    row["identical"] = bool(torch.equal(outs[False].view(torch.int16), outs[True].view(torch.int16)))
    return row


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode32k", "decode128k", "prefill"], default=None,
                    help="run one section only (profiling)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="one launch of each kernel plus a calibration copy, for rocprofv3 --pmc")
    ap.add_argument("--calibration", action="store_true",
                    help="time the offline calibration path (layer-pair similarities, DP, head maps)")
    ap.add_argument("--dtype", choices=["bf16", "f16"], default="bf16",
                    help="element type of q, k, v and outputs (the workloads are defined in bf16)")
    ap.add_argument("--paged", action="store_true",
                    help="time decode and the reuse prefill over paged KV caches against contiguous caches")
    args = ap.parse_args()
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

    sections = ["decode32k", "decode128k", "prefill"] if args.only is None else [args.only]
    log("building workloads", sections)
    t_build = time.perf_counter()
    work = {}
    if "decode32k" in sections or not args.no_cpu_baseline:
        work["decode32k"] = build_decode(configs.LLAMA_DECODE_32K, torch, K, synth, configs, args.dtype)
    if "decode128k" in sections:
        work["decode128k"] = build_decode(configs.LLAMA_DECODE_128K, torch, K, synth, configs, args.dtype)
    if "prefill" in sections:
        work["prefill"] = build_prefill(torch, K, synth, configs, args.dtype)
    torch.cuda.synchronize()
    log("built in %.1f s" % (time.perf_counter() - t_build))

    def step():
        marks = {}
        for s in sections:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            work[s]["run"]()
            e1.record()
            marks[s] = (e0, e1)
        return marks

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log("warmup step %d done" % i)

    # pick the kernel with the largest share of one step, then time it live
    for kid in range(8):
        K.kascade_kernel_timer_enable(kid, True)
    step()
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
    dom_ms, dom_n = K.kascade_kernel_timer_read(dom)
    K.kascade_kernel_timer_enable(dom, False)
    log("timed %d steps in %.3f s" % (args.steps, wall))

    sec_ms = {s: float(np.mean([m[s][0].elapsed_time(m[s][1]) for m in all_marks])) for s in sections}

    comps = {}
    for s in ("decode32k", "decode128k"):
        if s not in sections:
            continue
        w = work[s]
        L = w["cfg"].n_layers
        by = w["n_anchor"] * w["bytes_anchor"] + w["n_reuse"] * w["bytes_reuse"]
        # per-kind breakdown outside the timed steps
        per = {}
        for kind, n in (("anchor", w["n_anchor"]), ("reuse", w["n_reuse"]), ("dense", L)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 5
            e0.record()
            for _ in range(reps):
                w["run"](kind)
            e1.record()
            torch.cuda.synchronize()
            per[kind] = e0.elapsed_time(e1) / reps / n * 1e3
        comps[s] = {
            "us_per_layer": sec_ms[s] * 1e3 / L,
            "GBps": by / (sec_ms[s] * 1e-3) / 1e9,
            "hbm_frac": by / (sec_ms[s] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "anchor_us": per["anchor"], "reuse_us": per["reuse"],
            "anchor_GBps": w["bytes_anchor"] / (per["anchor"] * 1e-6) / 1e9,
            "reuse_GBps": w["bytes_reuse"] / (per["reuse"] * 1e-6) / 1e9,
            "dense_us_per_layer": per["dense"],
            "dense_GBps": w["bytes_dense"] / (per["dense"] * 1e-6) / 1e9,
            "speedup_vs_dense": per["dense"] / (sec_ms[s] * 1e3 / L),
            "context": w["cfg"].ctx_len, "batch": w["cfg"].batch, "topk": w["cfg"].topk,
        }
    if "prefill" in sections:
        w = work["prefill"]
        rf = w["reuse_flops"]()
        fl = w["n_anchor"] * (w["flops_flash"] + w["flops_pool"]) + rf
        per = {}
        for kind, n in (("anchor", w["n_anchor"]), ("reuse", w["n_reuse"]), ("dense", 1)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            w["run"](kind)
            e1.record()
            torch.cuda.synchronize()
            per[kind] = e0.elapsed_time(e1) / n
        comps["prefill32k"] = {
            "ms": sec_ms["prefill"], "TFLOPs": fl / (sec_ms["prefill"] * 1e-3) / 1e12,
            "anchor_ms": per["anchor"], "reuse_ms": per["reuse"],
            "anchor_TFLOPs": (w["flops_flash"] + w["flops_pool"]) / (per["anchor"] * 1e-3) / 1e12,
            "reuse_TFLOPs": rf / w["n_reuse"] / (per["reuse"] * 1e-3) / 1e12,
            "mfma_frac": fl / (sec_ms["prefill"] * 1e-3) / 1e12 / MFMA16_PEAK_TFLOPS,
            "anchor_mfma_frac": (w["flops_flash"] + w["flops_pool"]) / (per["anchor"] * 1e-3) / 1e12
            / MFMA16_PEAK_TFLOPS,
            "dense_ms_per_layer": per["dense"],
            "dense_TFLOPs": w["flops_flash"] / (per["dense"] * 1e-3) / 1e12,
            "speedup_vs_dense": per["dense"] * w["cfg"].n_layers / sec_ms["prefill"],
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

    ms_per_step = wall * 1e3 / args.steps
    value = comps.get("decode32k", {}).get("us_per_layer")
    line = {
        "metric": METRIC, "value": value, "unit": "us/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": args.dtype, "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B-shaped attention, 32 layers, 32q/8kv heads, d=128, "
                               "anchors [0,2,8,13,14]: decode 32K ctx B=1 k=3264 + decode 128K ctx "
                               "B=4 k=13120 + prefill 32K tokens (tile 128, k_t min 256)",
                   "sections": sections},
        "components": comps, "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        line["cpu_baseline"] = cpu_baseline(work["decode32k"], torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

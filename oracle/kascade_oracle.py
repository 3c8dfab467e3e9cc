"""Plain fp64 CPU oracle for Kascade's anchor/reuse Top-k sparse attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never links, imports or calls it, and it imports nothing from the HIP
path: it takes NumPy arrays (the exact values the GPU is given, upcast to
float64) and returns NumPy arrays.

Sources.  The method is described on the web pages about the paper
"Kascade: A Practical Sparse Attention Method for Long-Context LLM Inference"
(arXiv 2512.16391).  Citations below name the page and its section:

* [Explainer] = the Japanese explainer page at 0h-n0.github.io titled
  "論文解説: Kascade — レイヤー間スパーシティ再利用による実用的長文脈LLM推論高速化".
  Its sections: "アンカーレイヤーと再利用レイヤー" (anchor / reuse layers),
  "レイヤー間類似度とアンカーレイヤー選択" (eq. sim and eq. w),
  "動的計画法（Algorithm 1）" (the DP recurrence), "ヘッドリマッピング" (head remap),
  "Top-k設定" (eq. k), "実装のポイント" (the implementation notes: 128-query
  prefill tiles).
* [Abstract] = the paper's abstract (fugumt.com and montaan.com pages):
  exact Top-k in anchor layers, reuse in intermediate layers, head-aware
  selection, tile-level operations in prefill and decode.

Readings adopted where the pages are silent:
pooling is the SUM of post-softmax probabilities over the pooled queries;
query head h uses KV head h // G; softmax scale 1/sqrt(d); a reuse layer uses
the nearest preceding anchor; sparse softmax is renormalised over the selected
keys; ties in Top-k go to the lower index; index lists are returned ascending;
the k rule rounds 10% of n to the nearest multiple of 64 (halves up).

Every function here follows the definition as written: no blocking, fusion or
reordering beyond what the definition states.  Parity of each function is
pinned by tests under ``tests/test_oracle_*.py`` (library routines, closed
forms, invariants and brute force); none is "parity unpinned" except the
absolute end-to-end values, which the pages do not print.
"""
from __future__ import annotations

import itertools
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "topk_for_len", "prefill_tile_k", "kv_head_of", "anchor_of",
    "dense_decode", "pool_decode", "topk_full_sort", "sparse_decode",
    "anchor_decode", "reuse_decode",
    "dense_prefill", "dense_prefill_rows", "tile_pool", "tile_pool_one",
    "tile_topk", "sparse_prefill", "sparse_prefill_rows",
    "anchor_prefill", "reuse_prefill",
    "sim", "head_similarity", "head_map_from_similarity", "remapped_layer_similarity",
    "layer_weight", "weighted_similarity", "dp_select_anchors",
    "brute_force_anchors", "coverage_score",
    "run_decode_layerstack", "index_sets_agree",
]


# ---------------------------------------------------------------------------
# small helpers
# ---------------------------------------------------------------------------

def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if not np.issubdtype(a.dtype, np.floating):
        raise TypeError("oracle expects floating point arrays")
    a = a.astype(np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("oracle input holds a non-finite value")
    return a


def _scale(d: int, scale: Optional[float]) -> float:
    # Reading: SDPA's default softmax scale 1/sqrt(head_dim).
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def kv_head_of(h: int, group: int) -> int:
    """Reading for GQA: consecutive query heads share one KV head, h -> h // G."""
    return h // group


def anchor_of(layer: int, anchors: Sequence[int]) -> int:
    """The nearest anchor at or before ``layer``.

    [Explainer] "アンカーレイヤーと再利用レイヤー": a reuse layer takes the indices
    of the preceding anchor layer; in the DP each segment [i, j) is served by
    anchor i.
    """
    prev = [a for a in anchors if a <= layer]
    if not prev:
        raise ValueError("layer %d has no preceding anchor" % layer)
    return max(prev)


# ---------------------------------------------------------------------------
# k rule
# ---------------------------------------------------------------------------

def topk_for_len(n: int, pct: int = 10, round_to: int = 64, k_min: int = 128) -> int:
    """k for a row of n keys.

    [Explainer] "Top-k設定": k = min(max(0.1*N, 128), N).  The configured
    workloads print k=3264 at N=32768 and k=13120 at N=131072, i.e. 10% of N
    rounded to the NEAREST multiple of 64 (floor would give 13056, ceiling
    3328); halves round up.  Integer arithmetic only.
    """
    if n < 0:
        raise ValueError("negative length")
    r = int(round_to)
    tenth = r * ((n * pct + 50 * r) // (100 * r))
    return int(min(n, max(k_min, tenth)))


def prefill_tile_k(t: int, n: int, tile: int = 128, pct: int = 10,
                   round_to: int = 64, k_min: int = 256) -> Tuple[int, int]:
    """(P_t, k_t) for prefill query tile t: the causal prefix P_t that the last
    row of the tile sees, and its k (eq. k with the prefill minimum of 256)."""
    p = min(n, tile * (t + 1))
    return p, topk_for_len(p, pct, round_to, k_min)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def dense_decode(q, k, v, scale=None):
    """Exact dense decode attention for one query per (batch, head).

    q [B,Hq,d]; k, v [B,Hkv,N,d].  Returns (out [B,Hq,d], lse [B,Hq],
    p [B,Hq,N]) with s_j = scale*q.k_j, lse = log sum_j exp(s_j), p_j =
    exp(s_j - lse), out = sum_j p_j v_j.  No mask: the query sees all N keys.
    [Explainer] "アンカーレイヤーと再利用レイヤー": anchor layers compute full
    attention; P is the post-softmax distribution of eq. sim.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, d = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    G = Hq // Hkv
    sc = _scale(d, scale)
    out = np.zeros((B, Hq, v.shape[-1]))
    lse = np.zeros((B, Hq))
    p = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, G)
            s = sc * (k[b, g] @ q[b, h])
            m = s.max()
            lse[b, h] = m + math.log(np.exp(s - m).sum())
            p[b, h] = np.exp(s - lse[b, h])
            out[b, h] = p[b, h] @ v[b, g]
    return out, lse, p


def pool_decode(p, n_kv_heads: int):
    """Head-aware pooling of post-softmax probabilities per KV head.

    pooled[b,g,j] = sum over the query heads h of group g of p[b,h,j].
    [Abstract] (head-aware Top-k) and [Explainer] "ヘッドリマッピング" (indices are
    kept per KV head).  Reading: the pooling operator is a sum.
    """
    p = _f64(p)
    B, Hq, N = p.shape
    G = Hq // n_kv_heads
    pooled = np.zeros((B, n_kv_heads, N))
    for h in range(Hq):
        pooled[:, kv_head_of(h, G)] += p[:, h]
    return pooled


def topk_full_sort(scores, k: int) -> np.ndarray:
    """Exact Top-k by a full sort: the k largest values, ties to the lower
    index, returned in ascending index order (int64).

    [Abstract]: anchors compute EXACT Top-k indices.  Order the positions by
    (-score, index) with a full lexicographic sort and keep the first k.
    -0.0 compares equal to +0.0 here, so the two are one key.
    """
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    if not np.all(np.isfinite(s)):
        raise ValueError("non-finite score")
    n = s.shape[0]
    k = int(min(max(k, 0), n))
    idx = np.arange(n)
    order = np.lexsort((idx, -s))  # primary key -s, secondary key index
    return np.sort(order[:k]).astype(np.int64)


def sparse_decode(q, k, v, idx, head_map=None, scale=None):
    """Decode attention over a selected key set, softmax renormalised over it.

    q [B,Hq,d]; k, v [B,Hkv,N,d] (this layer's cache); idx [B,Hkv_a,kk] the
    anchor's index lists; head_map[g] names the anchor KV head whose list KV
    head g uses (identity if None).  For query head h, J = idx[b, head_map[h//G]]
    and out = sum_{j in J} softmax_J(scale*q.k_j) v_j.
    [Explainer] "アンカーレイヤーと再利用レイヤー" (attention on the selected keys
    only) and "ヘッドリマッピング" (per-KV-head remap).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    idx = np.asarray(idx)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = _scale(d, scale)
    hm = list(range(Hkv)) if head_map is None else [int(x) for x in head_map]
    out = np.zeros((B, Hq, v.shape[-1]))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, G)
            J = idx[b, hm[g]]
            J = J[J >= 0]
            if J.size == 0:
                raise ValueError("empty selected set")
            s = sc * (k[b, g, J] @ q[b, h])
            m = s.max()
            lse[b, h] = m + math.log(np.exp(s - m).sum())
            w = np.exp(s - lse[b, h])
            out[b, h] = w @ v[b, g, J]
    return out, lse


def anchor_decode(q, k, v, topk: int, scale=None):
    """One anchor decode layer: dense output, pooled scores, Top-k per KV head.

    Returns (out, lse, pooled [B,Hkv,N], idx [B,Hkv,topk] ascending)."""
    out, lse, p = dense_decode(q, k, v, scale)
    Hkv = np.asarray(k).shape[1]
    pooled = pool_decode(p, Hkv)
    B = pooled.shape[0]
    idx = np.zeros((B, Hkv, min(topk, pooled.shape[2])), dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            idx[b, g] = topk_full_sort(pooled[b, g], topk)
    return out, lse, pooled, idx


def reuse_decode(q, k, v, anchor_idx, head_map, scale=None):
    """One reuse decode layer: the anchor's lists through the head remap."""
    return sparse_decode(q, k, v, anchor_idx, head_map, scale)[0]


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def dense_prefill_rows(q, k, v, b: int, h: int, rows: Sequence[int], scale=None):
    """Causal dense attention for selected query rows of one (batch, head).

    q [B,Hq,N,d]; k, v [B,Hkv,N,d].  Row r sees keys 0..r.  Returns
    (out [len(rows), d], lse [len(rows)], p [len(rows), N] zero beyond r)."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    Hq, N, d = q.shape[1], q.shape[2], q.shape[3]
    Hkv = k.shape[1]
    g = kv_head_of(h, Hq // Hkv)
    sc = _scale(d, scale)
    rows = list(rows)
    out = np.zeros((len(rows), v.shape[-1]))
    lse = np.zeros(len(rows))
    p = np.zeros((len(rows), N))
    kg = _f64(k[b, g])
    vg = _f64(v[b, g])
    for i, r in enumerate(rows):
        s = sc * (kg[: r + 1] @ _f64(q[b, h, r]))
        m = s.max()
        lse[i] = m + math.log(np.exp(s - m).sum())
        p[i, : r + 1] = np.exp(s - lse[i])
        out[i] = p[i, : r + 1] @ vg[: r + 1]
    return out, lse, p


def dense_prefill(q, k, v, scale=None):
    """Causal dense prefill attention over all rows (small N only).

    Returns (out [B,Hq,N,d], lse [B,Hq,N])."""
    q = np.asarray(q)
    B, Hq, N, d = q.shape
    out = np.zeros((B, Hq, N, np.asarray(v).shape[-1]))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            o, l, _ = dense_prefill_rows(q, k, v, b, h, range(N), scale)
            out[b, h], lse[b, h] = o, l
    return out, lse


def tile_pool_one(q, k, b: int, t: int, g: int, tile: int = 128, scale=None):
    """Tile-level pooled post-softmax scores for one (batch, tile, KV head).

    pooled[j] = sum over the query heads h of group g and the rows r of tile t
    of P[h, r, j], for j < P_t, with P[h, r, j] = 0 for j > r (causal).
    [Abstract] (tile-level operations in prefill), [Explainer] "実装のポイント"
    (128-query tiles) and "アンカーレイヤーと再利用レイヤー" (post-softmax
    distribution).  Reading: the pooling operator is a sum.
    """
    q = np.asarray(q)
    Hq, N = q.shape[1], q.shape[2]
    Hkv = np.asarray(k).shape[1]
    G = Hq // Hkv
    lo, hi = tile * t, min(N, tile * (t + 1))
    P_t = hi
    pooled = np.zeros(P_t)
    for h in range(g * G, (g + 1) * G):
        _, _, p = dense_prefill_rows(q, k, k, b, h, range(lo, hi), scale)
        pooled += p[:, :P_t].sum(axis=0)
    return pooled


def tile_pool(q, k, tile: int = 128, scale=None):
    """All tiles: list over (b, t, g) of pooled rows (ragged, length P_t)."""
    q = np.asarray(q)
    B, N = q.shape[0], q.shape[2]
    Hkv = np.asarray(k).shape[1]
    T = -(-N // tile)
    return [[[tile_pool_one(q, k, b, t, g, tile, scale) for g in range(Hkv)]
             for t in range(T)] for b in range(B)]


def tile_topk(pooled_rows, n: int, tile: int = 128, pct: int = 10,
              round_to: int = 64, k_min: int = 256) -> np.ndarray:
    """Exact Top-k of every pooled tile row with the per-tile k_t.

    Returns int64 [B, T, Hkv, k_max], ascending, padded with -1 after k_t,
    where k_max is the k of the last tile."""
    B = len(pooled_rows)
    T = len(pooled_rows[0])
    Hkv = len(pooled_rows[0][0])
    k_max = prefill_tile_k(T - 1, n, tile, pct, round_to, k_min)[1]
    idx = -np.ones((B, T, Hkv, k_max), dtype=np.int64)
    for b in range(B):
        for t in range(T):
            _, k_t = prefill_tile_k(t, n, tile, pct, round_to, k_min)
            for g in range(Hkv):
                idx[b, t, g, :k_t] = topk_full_sort(pooled_rows[b][t][g], k_t)
    return idx


def sparse_prefill_rows(q, k, v, tile_idx, head_map, b: int, h: int,
                        rows: Sequence[int], tile: int = 128, scale=None):
    """Sparse causal prefill attention for selected rows of one (batch, head).

    Row r of tile t = r // tile attends to J = {j in tile_idx[b, t,
    head_map[h // G]] : j >= 0 and j <= r}, softmax renormalised over J.
    [Explainer] "アンカーレイヤーと再利用レイヤー" and "ヘッドリマッピング".
    Reading: the causal mask applies inside the selected set; no forced window.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    Hq, d = q.shape[1], q.shape[3]
    Hkv = k.shape[1]
    g = kv_head_of(h, Hq // Hkv)
    src = int(head_map[g]) if head_map is not None else g
    sc = _scale(d, scale)
    kg = _f64(k[b, g])
    vg = _f64(v[b, g])
    rows = list(rows)
    out = np.zeros((len(rows), v.shape[-1]))
    for i, r in enumerate(rows):
        J = np.asarray(tile_idx[b, r // tile, src])
        J = J[(J >= 0) & (J <= r)]
        if J.size == 0:
            raise ValueError("row %d has an empty selected set" % r)
        s = sc * (kg[J] @ _f64(q[b, h, r]))
        m = s.max()
        w = np.exp(s - m)
        w /= w.sum()
        out[i] = w @ vg[J]
    return out


def sparse_prefill(q, k, v, tile_idx, head_map=None, tile: int = 128, scale=None):
    """Sparse causal prefill over all rows (small N only). out [B,Hq,N,d]."""
    q = np.asarray(q)
    B, Hq, N, d = q.shape
    out = np.zeros((B, Hq, N, np.asarray(v).shape[-1]))
    for b in range(B):
        for h in range(Hq):
            out[b, h] = sparse_prefill_rows(q, k, v, tile_idx, head_map, b, h,
                                            range(N), tile, scale)
    return out


def anchor_prefill(q, k, v, tile: int = 128, pct: int = 10, round_to: int = 64,
                   k_min: int = 256, scale=None):
    """One anchor prefill layer: (dense out, lse, pooled rows, tile idx)."""
    out, lse = dense_prefill(q, k, v, scale)
    pooled = tile_pool(q, k, tile, scale)
    idx = tile_topk(pooled, np.asarray(q).shape[2], tile, pct, round_to, k_min)
    return out, lse, pooled, idx


def reuse_prefill(q, k, v, anchor_tile_idx, head_map, tile: int = 128, scale=None):
    """One reuse prefill layer."""
    return sparse_prefill(q, k, v, anchor_tile_idx, head_map, tile, scale)


# ---------------------------------------------------------------------------
# offline anchor selection: eq. sim, eq. w, the weighted matrix and the DP
# ---------------------------------------------------------------------------

def sim(p_a, p_b, k: int) -> float:
    """Cross-layer similarity of one query (or pooled row).

    [Explainer] "レイヤー間類似度とアンカーレイヤー選択", eq. sim: the mass that
    layer b's distribution puts on layer a's Top-k set, divided by the mass it
    puts on its own Top-k set.
    """
    p_a = _f64(p_a).reshape(-1)
    p_b = _f64(p_b).reshape(-1)
    I_a = topk_full_sort(p_a, k)
    I_b = topk_full_sort(p_b, k)
    return float(p_b[I_a].sum() / p_b[I_b].sum())


def head_similarity(pooled_a, pooled_b, k: int) -> np.ndarray:
    """Per-KV-head cross-layer similarity, averaged over samples.

    pooled_a, pooled_b: [S, Hkv, N] pooled post-softmax rows of layers a and b
    for the same S calibration queries.  Returns M [Hkv_a, Hkv_b] with
    M[ga, gb] = mean over samples s of sim(pooled_a[s, ga], pooled_b[s, gb], k):
    [Explainer] eq. sim applied to every pair of KV heads, the quantity that
    section "ヘッドリマッピング" maximises to pair each head of a reuse layer with
    a head of its anchor.  Reading: samples are averaged with equal weight."""
    pa = _f64(pooled_a)
    pb = _f64(pooled_b)
    S, Ha = pa.shape[0], pa.shape[1]
    Hb = pb.shape[1]
    M = np.zeros((Ha, Hb))
    for ga in range(Ha):
        for gb in range(Hb):
            M[ga, gb] = sum(sim(pa[s, ga], pb[s, gb], k) for s in range(S)) / S
    return M


def head_map_from_similarity(M) -> np.ndarray:
    """[Explainer] "ヘッドリマッピング": each KV head gb of the reuse layer takes
    the anchor KV head with the largest similarity M[ga, gb]; ties go to the
    lower ga.  Returns int32 [Hkv_b]."""
    M = _f64(M)
    out = np.zeros(M.shape[1], dtype=np.int32)
    for gb in range(M.shape[1]):
        best = 0
        for ga in range(1, M.shape[0]):
            if M[ga, gb] > M[best, gb]:
                best = ga
        out[gb] = best
    return out


def remapped_layer_similarity(M) -> float:
    """Layer-level similarity of (anchor a, layer b) once b's heads are
    remapped: the mean over b's KV heads of their best similarity.  Reading
    of [Explainer] "レイヤー間類似度とアンカーレイヤー選択" together with
    "ヘッドリマッピング": a reuse layer always runs with the remap, so the
    similarity that selects anchors is the remapped one."""
    M = _f64(M)
    hm = head_map_from_similarity(M)
    return float(np.mean([M[hm[gb], gb] for gb in range(M.shape[1])]))


def layer_weight(x, y) -> float:
    """[Explainer] eq. w: w_l = 1 - cosine(x_l, y_l), x_l / y_l the layer's
    input / output hidden states.  Rows of x and y are tokens; reading: the
    per-token cosine is averaged over tokens.  A zero vector raises."""
    x = _f64(x).reshape(-1, np.asarray(x).shape[-1])
    y = _f64(y).reshape(-1, np.asarray(y).shape[-1])
    nx = np.sqrt((x * x).sum(axis=1))
    ny = np.sqrt((y * y).sum(axis=1))
    if np.any(nx == 0) or np.any(ny == 0):
        raise ValueError("cosine of a zero vector is undefined")
    cos = (x * y).sum(axis=1) / (nx * ny)
    return float(1.0 - cos.mean())


def weighted_similarity(sim_bar, w) -> np.ndarray:
    """S[a][b] = w_b * sim_bar[a][b] for b >= a (0 below the diagonal).

    Reading of [Explainer] "動的計画法（Algorithm 1）": S is the similarity
    matrix weighted by the importance of the approximated layer b."""
    sim_bar = _f64(sim_bar)
    w = _f64(w).reshape(-1)
    L = sim_bar.shape[0]
    S = np.zeros((L, L))
    for a in range(L):
        for b in range(a, L):
            S[a, b] = w[b] * sim_bar[a, b]
    return S


def dp_select_anchors(S, M: int) -> Tuple[List[int], float]:
    """Algorithm 1: choose M anchor layers out of L maximising total similarity.

    [Explainer] "動的計画法（Algorithm 1）":
      dp[m][j] = max over i in [m-1, j-1] of dp[m-1][i] + sum_{l=i}^{j-1} S[i][l],
    dp[0][0] = 0 and dp[0][j>0] = -inf, answer dp[M][L], anchors recovered by
    backtracking through the maximising i.  Segment [i, j) is served by
    anchor i.  Ties keep the smallest i.  O(M L^2) with row prefix sums.
    """
    S = _f64(S)
    L = S.shape[0]
    if not 1 <= M <= L:
        raise ValueError("need 1 <= M <= L")
    # pref[i][j] = sum_{l=i}^{j-1} S[i][l]
    pref = np.zeros((L, L + 1))
    for i in range(L):
        acc = 0.0
        for j in range(i, L):
            acc += S[i, j]
            pref[i, j + 1] = acc
    NEG = -math.inf
    dp = np.full((M + 1, L + 1), NEG)
    arg = np.full((M + 1, L + 1), -1, dtype=np.int64)
    dp[0, 0] = 0.0
    for m in range(1, M + 1):
        for j in range(m, L + 1):
            best, best_i = NEG, -1
            for i in range(m - 1, j):
                if dp[m - 1, i] == NEG:
                    continue
                val = dp[m - 1, i] + pref[i, j]
                if val > best:
                    best, best_i = val, i
            dp[m, j], arg[m, j] = best, best_i
    anchors = []
    j = L
    for m in range(M, 0, -1):
        i = int(arg[m, j])
        anchors.append(i)
        j = i
    anchors.reverse()
    return anchors, float(dp[M, L])


def coverage_score(S, anchors: Sequence[int]) -> float:
    """Total similarity of an anchor set: sum_l S[a(l)][l]."""
    S = _f64(S)
    return float(sum(S[anchor_of(l, anchors), l] for l in range(S.shape[0])))


def brute_force_anchors(S, M: int) -> Tuple[List[int], float]:
    """Enumerate every M-subset of layers containing layer 0 (test helper)."""
    S = _f64(S)
    L = S.shape[0]
    best, best_set = -math.inf, None
    for rest in itertools.combinations(range(1, L), M - 1):
        cand = [0] + list(rest)
        val = coverage_score(S, cand)
        if val > best:
            best, best_set = val, cand
    return best_set, best


# ---------------------------------------------------------------------------
# layer stack and comparison rule
# ---------------------------------------------------------------------------

def run_decode_layerstack(layers: Sequence[Dict], anchors: Sequence[int],
                          head_maps: Dict[int, Sequence[int]], topk: int,
                          scale=None):
    """Decode through a stack: anchors run dense attention and select; reuse
    layers take their nearest preceding anchor's lists through head_maps[l].

    layers[l] = {"q":..., "k":..., "v":...}.  Returns (outs, idx_by_anchor)."""
    outs, idx_by_anchor = [], {}
    for l, lay in enumerate(layers):
        if l in anchors:
            out, _, _, idx = anchor_decode(lay["q"], lay["k"], lay["v"], topk, scale)
            idx_by_anchor[l] = idx
        else:
            a = anchor_of(l, anchors)
            out = reuse_decode(lay["q"], lay["k"], lay["v"], idx_by_anchor[a],
                               head_maps[l], scale)
        outs.append(out)
    return outs, idx_by_anchor


def index_sets_agree(sel, ref_idx, ref_scores, rel: float = 1e-5) -> Tuple[bool, int]:
    """Acceptance rule for end-to-end index sets.

    Every element of the symmetric difference between ``sel`` and ``ref_idx``
    must have a reference score within ``rel`` (relative) of the reference's
    k-th value.  Returns (ok, size of symmetric difference)."""
    sel = set(int(x) for x in np.asarray(sel).reshape(-1) if x >= 0)
    ref = [int(x) for x in np.asarray(ref_idx).reshape(-1) if x >= 0]
    s = np.asarray(ref_scores, dtype=np.float64)
    kth = s[ref].min() if ref else 0.0
    diff = sel.symmetric_difference(ref)
    tol = rel * abs(kth)
    ok = len(sel) == len(ref) and all(abs(s[j] - kth) <= tol for j in diff)
    return ok, len(diff)

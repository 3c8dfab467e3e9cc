"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only draws numbers: it holds none of the attention method's
arithmetic.  Both sides are handed the very tensors produced here (the oracle
gets them copied to host memory and upcast exactly to float64).

Workload shape (stand-in for the pages' long-context model workloads, which
need weights and datasets that are not available):
  * Q, K, V entries are N(0, 1), drawn in fp32 and rounded to the working
    dtype (bf16 and fp16 rounding is round-to-nearest-even, done by torch).
  * About 10% of key positions per KV head are "heavy": their keys get a
    planted component alpha * u along a direction u that the queries share,
    so that they carry most of the softmax mass (the pages report that about
    10% of keys hold about 95% of the post-softmax mass).
  * Heavy sets drift between consecutive layers (a fraction `drift` of the
    members is replaced per layer), mimicking the reported cross-layer
    stability of high-weight keys.
  * A reuse layer's KV head g inherits the lineage of anchor KV head
    head_map[g], so the supplied head map is the right remap by construction.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in key]))


def _tgen(device, *key: int) -> torch.Generator:
    g = torch.Generator(device=device)
    h = 0x9E3779B97F4A7C15
    for k in key:
        h = (h ^ (int(k) & 0xFFFFFFFFFFFFFFFF)) * 0x100000001B3 & 0xFFFFFFFFFFFFFFFF
    g.manual_seed(h & 0x7FFFFFFFFFFFFFFF)
    return g


# ---------------------------------------------------------------------------
# index structure: heavy lineages, head maps, anchors
# ---------------------------------------------------------------------------

def heavy_lineages(seed: int, n_layers: int, n_kv: int, n: int, n_heavy: int,
                   drift: float) -> List[List[np.ndarray]]:
    """lin[l][c]: sorted heavy positions of lineage c at layer l."""
    lin: List[List[np.ndarray]] = []
    n_swap = int(round(drift * n_heavy))
    for c in range(n_kv):
        r = _rng(seed, 11, c)
        cur = np.sort(r.choice(n, size=n_heavy, replace=False))
        per_layer = [cur]
        for _ in range(1, n_layers):
            keep = np.sort(r.choice(cur.size, size=cur.size - n_swap, replace=False))
            members = np.zeros(n, dtype=bool)
            members[cur] = True
            outside = np.flatnonzero(~members)
            new = r.choice(outside, size=n_swap, replace=False)
            cur = np.sort(np.concatenate([cur[keep], new]))
            per_layer.append(cur)
        for l, s in enumerate(per_layer):
            if c == 0:
                lin.append([])
            lin[l].append(s)
    return lin


def head_maps(seed: int, n_layers: int, anchors: Sequence[int], n_kv: int,
              kind: str) -> Dict[int, np.ndarray]:
    """Per reuse layer: int32 [n_kv] map to anchor KV heads."""
    maps: Dict[int, np.ndarray] = {}
    for l in range(n_layers):
        if l in anchors:
            continue
        r = _rng(seed, 23, l)
        if kind == "identity":
            m = np.arange(n_kv)
        elif kind == "perm":
            m = r.permutation(n_kv)
        elif kind == "learned":
            m = np.arange(n_kv)
            for g in range(n_kv):
                if r.random() >= 0.5 and n_kv > 1:
                    others = [x for x in range(n_kv) if x != g]
                    m[g] = others[int(r.integers(len(others)))]
        else:
            raise ValueError(kind)
        maps[l] = m.astype(np.int32)
    return maps


def layer_heavy_sets(lin, layer: int, anchors: Sequence[int], maps) -> List[np.ndarray]:
    """Heavy positions of each KV head of ``layer``: anchors use lineage g,
    reuse layers use lineage head_map[g]."""
    n_kv = len(lin[layer])
    if layer in anchors:
        return [lin[layer][g] for g in range(n_kv)]
    return [lin[layer][int(maps[layer][g])] for g in range(n_kv)]


def similarity_matrix(seed: int, n_layers: int) -> np.ndarray:
    """Synthetic weighted similarity matrix S (weights folded in):
    S[a][a] = 1; for b > a, U(0.95, 1.0) - 0.01*(b-a-1), clamped at 0."""
    r = _rng(seed, 31)
    S = np.zeros((n_layers, n_layers))
    for a in range(n_layers):
        S[a, a] = 1.0
        for b in range(a + 1, n_layers):
            S[a, b] = max(0.0, r.uniform(0.95, 1.0) - 0.01 * (b - a - 1))
    return S


# ---------------------------------------------------------------------------
# dense tensors
# ---------------------------------------------------------------------------

def _randn(shape, gen, device) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def decode_layer(seed: int, layer: int, batch: int, n_q: int, n_kv: int, d: int,
                 n: int, heavy: Sequence[np.ndarray], alpha: float, dtype: str,
                 device="cpu", n_max: Optional[int] = None):
    """One decode layer: q [B,Hq,d], k/v [B,Hkv,n_max,d] (first n rows filled).

    Heavy keys of KV head g get alpha * u added, u the unit vector along the
    sum of the group's queries."""
    n_max = n_max or n
    G = n_q // n_kv
    gen = _tgen(device, seed, 101, layer)
    q = _randn((batch, n_q, d), gen, device)
    kk = _randn((batch, n_kv, n, d), gen, device)
    v = _randn((batch, n_kv, n, d), gen, device)
    u = q.view(batch, n_kv, G, d).sum(dim=2)
    u = u / u.norm(dim=-1, keepdim=True)
    for g in range(n_kv):
        pos = torch.as_tensor(heavy[g], device=device, dtype=torch.long)
        kk[:, g].index_add_(1, pos, (alpha * u[:, g]).unsqueeze(1).expand(batch, pos.numel(), d).contiguous())
    td = _DT[dtype]
    if n_max > n:
        kf = torch.zeros((batch, n_kv, n_max, d), device=device, dtype=td)
        vf = torch.zeros((batch, n_kv, n_max, d), device=device, dtype=td)
        kf[:, :, :n] = kk.to(td)
        vf[:, :, :n] = v.to(td)
        return q.to(td), kf, vf
    return q.to(td), kk.to(td), v.to(td)


def prefill_layer(seed: int, layer: int, batch: int, n_q: int, n_kv: int, d: int,
                  n: int, heavy: Sequence[np.ndarray], alpha: float, gamma: float,
                  dtype: str, device="cpu", n_max: Optional[int] = None):
    """One prefill layer: q [B,Hq,n,d], k/v [B,Hkv,n_max,d].

    Per KV head a seeded unit direction u: queries are z + gamma*u, heavy keys
    get alpha*u added."""
    n_max = n_max or n
    G = n_q // n_kv
    gen = _tgen(device, seed, 202, layer)
    u = _unit_rows(_randn((n_kv, d), gen, device))
    td = _DT[dtype]
    q = torch.empty((batch, n_q, n, d), device=device, dtype=td)
    k = torch.zeros((batch, n_kv, n_max, d), device=device, dtype=td)
    v = torch.zeros((batch, n_kv, n_max, d), device=device, dtype=td)
    for h in range(n_q):
        z = _randn((batch, n, d), gen, device)
        z += gamma * u[h // G]
        q[:, h] = z.to(td)
    for g in range(n_kv):
        kk = _randn((batch, n, d), gen, device)
        pos = torch.as_tensor(heavy[g], device=device, dtype=torch.long)
        kk.index_add_(1, pos, (alpha * u[g]).expand(batch, pos.numel(), d).contiguous())
        k[:, g, :n] = kk.to(td)
        v[:, g, :n] = _randn((batch, n, d), gen, device).to(td)
    return q, k, v


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def prefill_directions(seed: int, layer: int, n_kv: int, d: int, device="cpu") -> torch.Tensor:
    """The per-KV-head unit directions u [n_kv, d] that prefill_layer plants
    (the first draw of the same generator)."""
    return _unit_rows(_randn((n_kv, d), _tgen(device, seed, 202, layer), device))


def decode_step(seed: int, layer: int, step: int, batch: int, n_q: int, n_kv: int, d: int,
                u: torch.Tensor, gamma: float, dtype: str, device="cpu"):
    """Inputs of one generated token after a prefill: the query [B,Hq,d] is
    z + gamma*u[h // G] and the appended K and V rows [B,Hkv,d] are N(0,1)."""
    G = n_q // n_kv
    gen = _tgen(device, seed, 505, layer, step)
    q = _randn((batch, n_q, d), gen, device) + gamma * u.repeat_interleave(G, dim=0)
    k_row = _randn((batch, n_kv, d), gen, device)
    v_row = _randn((batch, n_kv, d), gen, device)
    td = _DT[dtype]
    return q.to(td), k_row.to(td), v_row.to(td)


def score_rows(seed: int, rows: int, n: int, kind: str = "normal", device="cpu") -> torch.Tensor:
    """fp32 score rows for the Top-k select tests.

    kind: "normal" (continuous), "ties" (values from a small set so that many
    ties cross the k-th value), "const" (one value), "signed" (mixed signs,
    including -0.0 and +0.0), "pooled" (non-negative, heavy-tailed)."""
    gen = _tgen(device, seed, 303, rows, n)
    if kind == "normal":
        x = torch.randn((rows, n), generator=gen, device=device)
    elif kind == "ties":
        x = torch.randint(0, 7, (rows, n), generator=gen, device=device).float() * 0.25
    elif kind == "const":
        x = torch.full((rows, n), 0.5, device=device)
    elif kind == "signed":
        x = torch.randint(-3, 4, (rows, n), generator=gen, device=device).float()
        zero = x == 0
        neg = torch.rand((rows, n), generator=gen, device=device) < 0.5
        x = torch.where(zero & neg, torch.full_like(x, -0.0), x)
    elif kind == "pooled":
        x = torch.exp(3.0 * torch.randn((rows, n), generator=gen, device=device)) * 1e-4
    else:
        raise ValueError(kind)
    return x.contiguous()


def random_index_lists(seed: int, batch: int, n_kv: int, n: int, k: int, device="cpu") -> torch.Tensor:
    """int32 [B,Hkv,k]: ascending random distinct positions in [0, n)."""
    r = _rng(seed, 41, batch, n_kv, n, k)
    out = np.zeros((batch, n_kv, k), dtype=np.int32)
    for b in range(batch):
        for g in range(n_kv):
            out[b, g] = np.sort(r.choice(n, size=k, replace=False))
    return torch.as_tensor(out, device=device)

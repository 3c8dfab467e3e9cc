"""The five workload definitions (shapes, anchors, k rule, generator settings).

These mirror the synthetic stand-ins for the pages' Llama-3.1-8B and Qwen3-8B
long-context workloads.  Nothing here computes any part of the method.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

LLAMA_ANCHORS: Tuple[int, ...] = (0, 2, 8, 13, 14)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "decode" | "prefill" | "e2e"
    dtype: str                # "f32" | "bf16" | "f16"
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int
    anchors: Tuple[int, ...]
    topk: int = 0             # decode k (0: k rule)
    head_map_kind: str = "perm"   # "identity" | "perm" | "learned"
    heavy_frac: float = 0.10
    n_heavy: int = 0          # 0: round(heavy_frac * ctx_len)
    drift: float = 0.05
    alpha: float = 0.0        # planted strength (decode: along the group's query direction)
    gamma: float = 4.0        # prefill: query component along the planted direction
    seed: int = 0
    tol: float = 2e-2
    tile: int = 128
    decode_steps: int = 0
    n_anchor_dp: int = 0      # e2e: number of anchors chosen by the DP

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def heavy(self) -> int:
        return self.n_heavy or int(round(self.heavy_frac * self.ctx_len))


TINY_DECODE = Workload("tiny-decode-f32", "decode", "f32", 2, 1, 4, 2, 64, 1024, (0,), topk=128,
                       head_map_kind="identity", n_heavy=64, drift=0.10, alpha=3.0, seed=1,
                       tol=1e-4)
LLAMA_DECODE_32K = Workload("llama8b-decode-32k", "decode", "bf16", 32, 1, 32, 8, 128, 32768,
                            LLAMA_ANCHORS, topk=3264, alpha=10.7, seed=2)
LLAMA_DECODE_128K = Workload("llama8b-decode-128k", "decode", "bf16", 32, 4, 32, 8, 128, 131072,
                             LLAMA_ANCHORS, topk=13120, alpha=10.7, seed=3)
LLAMA_PREFILL_32K = Workload("llama8b-prefill-32k", "prefill", "bf16", 32, 1, 32, 8, 128, 32768,
                             LLAMA_ANCHORS, alpha=17.5, seed=4)
QWEN3_E2E_64K = Workload("qwen3-8b-e2e-64k", "e2e", "bf16", 36, 1, 32, 8, 128, 65536, (),
                         head_map_kind="learned", alpha=17.5, seed=5, decode_steps=512,
                         n_anchor_dp=6)

WORKLOADS = {w.name: w for w in (TINY_DECODE, LLAMA_DECODE_32K, LLAMA_DECODE_128K,
                                 LLAMA_PREFILL_32K, QWEN3_E2E_64K)}

"""Host-side arithmetic of the benchmark (CPU only): the algorithmic bytes
and FLOPs that every roofline fraction divides by, pinned to the figures
worked out from the workload definitions (Llama-3.1-8B-shaped decode at
32K x 1 and 128K x 4, the 32K prefill), and the reuse-prefill FLOP count
against brute force on tiny lists."""
import dataclasses

import numpy as np
import torch

import bench
from long_context_anchor_amd import configs
from long_context_anchor_amd import kascade as K


def test_decode_bytes_match_the_worked_figures():
    # 2*B*Hkv*N*d*2 (K and V) + 2*B*Hq*d*2 (q in, out) + 4*B*Hkv*k (list)
    a, r, d = bench.decode_bytes(configs.LLAMA_DECODE_32K)
    assert a == 2 * 8 * 32768 * 128 * 2 + 2 * 32 * 128 * 2 + 4 * 8 * 3264 == 134_338_560
    assert r == 2 * 8 * 3264 * 128 * 2 + 2 * 32 * 128 * 2 + 4 * 8 * 3264 == 13_490_176
    assert d == 2 * 8 * 32768 * 128 * 2 + 2 * 32 * 128 * 2
    a, r, _ = bench.decode_bytes(configs.LLAMA_DECODE_128K)
    assert round(a / 1e6, 1) == 2149.2 and round(r / 1e6, 1) == 216.7


def test_prefill_flops_match_the_worked_figures():
    flash, pool = bench.prefill_flops(configs.LLAMA_PREFILL_32K)
    assert round(flash / 1e12, 3) == 8.796 and round(pool / 1e12, 3) == 4.398
    flash, pool = bench.prefill_flops(configs.QWEN3_E2E_64K)
    assert round((flash + pool) / 1e12, 2) == 52.78


def test_reuse_prefill_flops_brute_force():
    """Two 128-row tiles of a 256-token prompt, 2 KV heads of 2 query heads:
    the count equals 4*d*sum over query heads and rows of |{j in the row's
    tile list for head_map[g] : 0 <= j <= r}| counted by brute force."""
    N, Hkv, G, d = 256, 2, 2, 128
    rule = K.PREFILL_RULE
    T = N // rule.tile
    kmax = K.kascade_topk_for_len(N, rule)
    rng = np.random.default_rng(7)
    idx = np.full((1, T, Hkv, kmax), -1, dtype=np.int32)
    for t in range(T):
        P = min(N, rule.tile * (t + 1))
        kt = K.kascade_topk_for_len(P, rule)
        for g in range(Hkv):
            idx[0, t, g, :kt] = np.sort(rng.choice(P, kt, replace=False))
    maps = {1: [1, 0], 2: [0, 0]}
    got = bench.prefill_reuse_flops(torch, K, {0: torch.as_tensor(idx)}, {1: 0, 2: 0}, maps, [1, 2],
                                    N, Hkv, G, d)
    want = 0
    for l in (1, 2):
        for h in range(Hkv * G):
            src = maps[l][h // G]
            for r in range(N):
                lst = idx[0, r // rule.tile, src]
                want += int(((lst >= 0) & (lst <= r)).sum())
    assert got == 4.0 * d * want


def test_percentiles_and_host_info():
    st = bench.pct(np.arange(1, 101, dtype=float), 2.0)
    assert st["median"] == 101.0 and st["n"] == 100
    assert abs(st["p10"] - 2 * 10.9) < 1e-9 and abs(st["p90"] - 2 * 90.1) < 1e-9
    model, affinity, blas = bench.host_info()
    assert isinstance(model, str) and affinity >= 1 and blas >= 1

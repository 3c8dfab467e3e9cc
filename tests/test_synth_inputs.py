"""The seeded generators produce the workload statistics they claim (CPU).

The heavy-mass check uses the oracle's dense decode on a reduced context: about
10% of keys should carry about 95% of the softmax mass in the Llama-shaped
decode workloads (stand-in for the pages' reported intrinsic sparsity).
"""
import numpy as np

import oracle
from long_context_anchor_amd import configs, synth


def test_config_k_values_follow_the_k_rule():
    for c in (configs.LLAMA_DECODE_32K, configs.LLAMA_DECODE_128K):
        assert c.topk == oracle.topk_for_len(c.ctx_len)
    assert configs.TINY_DECODE.topk == oracle.topk_for_len(1024)


def test_lineage_drift_and_head_maps():
    lin = synth.heavy_lineages(2, 4, 3, 1000, 100, 0.05)
    for l in range(1, 4):
        for c in range(3):
            assert len(set(lin[l][c]) & set(lin[l - 1][c])) == 95
    maps = synth.head_maps(2, 32, configs.LLAMA_ANCHORS, 8, "perm")
    assert sorted(maps.keys()) == [l for l in range(32) if l not in configs.LLAMA_ANCHORS]
    for m in maps.values():
        assert sorted(m.tolist()) == list(range(8))
    learned = synth.head_maps(5, 36, (0,), 8, "learned")
    assert any(len(set(m.tolist())) < 8 for m in learned.values())


def test_decode_heavy_mass_near_95_percent():
    c = configs.LLAMA_DECODE_32K
    n, n_kv = 4096, 2
    lin = synth.heavy_lineages(9, 1, n_kv, n, int(0.1 * n), c.drift)
    q, k, v = synth.decode_layer(9, 0, 1, c.group * n_kv, n_kv, c.head_dim, n, lin[0], c.alpha, "bf16")
    _, _, p = oracle.dense_decode(q.float().numpy(), k.float().numpy(), v.float().numpy())
    mass = np.mean([p[0, h, lin[0][h // c.group]].sum() for h in range(c.group * n_kv)])
    assert 0.92 < mass < 0.98


def test_prefill_heavy_mass_near_95_percent():
    c = configs.LLAMA_PREFILL_32K
    n = 1024
    lin = synth.heavy_lineages(9, 1, 1, n, int(0.1 * n), c.drift)
    q, k, v = synth.prefill_layer(9, 0, 1, c.group, 1, c.head_dim, n, lin[0], c.alpha, c.gamma, "bf16")
    qn, kn, vn = q.float().numpy(), k.float().numpy(), v.float().numpy()
    masses = []
    for h in range(c.group):
        _, _, p = oracle.dense_prefill_rows(qn, kn, vn, 0, h, range(n // 2, n, 32))
        masses.append(p[:, lin[0][0]].sum(1).mean())
    assert 0.92 < np.mean(masses) < 0.98

"""The oracle's pins are discriminating: each test below plants one plausible
mistake in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a wrong tie rule or rounding) and checks that at least one of the
pin tests that cover that function then fails.  The mistakes are planted in
the oracle module only, on the CPU, for the duration of one test."""
import contextlib
import math

import numpy as np

import oracle
import oracle.kascade_oracle as ko
import test_oracle_attention as ta
import test_oracle_calibration as tc
import test_oracle_topk as tt

ORIG = {name: getattr(ko, name) for name in dir(ko) if not name.startswith("__")}


@contextlib.contextmanager
def planted(**fns):
    """Replace oracle functions (module and package names) for one test."""
    try:
        for name, fn in fns.items():
            setattr(ko, name, fn)
            if hasattr(oracle, name):
                setattr(oracle, name, fn)
        yield
    finally:
        for name in fns:
            setattr(ko, name, ORIG[name])
            if hasattr(oracle, name):
                setattr(oracle, name, ORIG[name])


def fails(pins):
    """True when at least one pin raises (an assertion or an error)."""
    for pin in pins:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure of the pin counts
            return True
    return False


def check(pins, **fns):
    assert not fails(pins), "the pins must pass on the unmodified oracle"
    with planted(**fns):
        assert fails(pins), "planted mistake not caught: %s" % ", ".join(fns)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def test_missing_softmax_scale_is_caught():
    check([ta.test_dense_decode_matches_library_sdpa, ta.test_dense_prefill_matches_causal_library_sdpa],
          _scale=lambda d, scale: 1.0 if scale is None else float(scale))


def test_interleaved_head_grouping_is_caught():
    def dense_decode(q, k, v, scale=None):
        q, k, v = ko._f64(q), ko._f64(k), ko._f64(v)
        B, Hq, d = q.shape
        Hkv, N = k.shape[1], k.shape[2]
        sc = ko._scale(d, scale)
        out, lse, p = np.zeros((B, Hq, v.shape[-1])), np.zeros((B, Hq)), np.zeros((B, Hq, N))
        for b in range(B):
            for h in range(Hq):
                g = h % Hkv                      # planted: heads interleaved over KV heads
                s = sc * (k[b, g] @ q[b, h])
                lse[b, h] = s.max() + math.log(np.exp(s - s.max()).sum())
                p[b, h] = np.exp(s - lse[b, h])
                out[b, h] = p[b, h] @ v[b, g]
        return out, lse, p
    check([ta.test_dense_decode_matches_library_sdpa], dense_decode=dense_decode)


def test_pooling_by_max_is_caught():
    def pool_decode(p, n_kv_heads):
        p = ko._f64(p)
        B, Hq, N = p.shape
        G = Hq // n_kv_heads
        pooled = np.zeros((B, n_kv_heads, N))
        for h in range(Hq):
            pooled[:, h // G] = np.maximum(pooled[:, h // G], p[:, h])   # planted: max, not sum
        return pooled
    check([ta.test_pool_decode_mass_and_group_one], pool_decode=pool_decode)


def test_sparse_softmax_not_renormalised_is_caught():
    def sparse_decode(q, k, v, idx, head_map=None, scale=None):
        _, lse_dense, _ = ORIG["dense_decode"](q, k, v, scale)
        q, k, v = ko._f64(q), ko._f64(k), ko._f64(v)
        idx = np.asarray(idx)
        B, Hq, d = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        hm = list(range(Hkv)) if head_map is None else [int(x) for x in head_map]
        out = np.zeros((B, Hq, v.shape[-1]))
        for b in range(B):
            for h in range(Hq):
                J = idx[b, hm[h // G]]
                s = ko._scale(d, scale) * (k[b, h // G, J] @ q[b, h])
                out[b, h] = np.exp(s - lse_dense[b, h]) @ v[b, h // G, J]   # planted: dense lse
        return out, lse_dense
    check([ta.test_sparse_decode_matches_masked_library_sdpa], sparse_decode=sparse_decode)


def test_ignored_head_map_is_caught():
    def sparse_decode(q, k, v, idx, head_map=None, scale=None):
        return ORIG["sparse_decode"](q, k, v, idx, None, scale)            # planted: no remap
    check([ta.test_sparse_decode_matches_masked_library_sdpa], sparse_decode=sparse_decode)


def test_causal_mask_off_by_one_is_caught():
    def dense_prefill_rows(q, k, v, b, h, rows, scale=None):
        q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
        Hq, N, d = q.shape[1], q.shape[2], q.shape[3]
        g = h // (Hq // k.shape[1])
        rows = list(rows)
        out, lse, p = np.zeros((len(rows), v.shape[-1])), np.zeros(len(rows)), np.zeros((len(rows), N))
        for i, r in enumerate(rows):
            e = min(N, r + 2)                                                # planted: sees key r + 1
            s = ko._scale(d, scale) * (ko._f64(k[b, g])[:e] @ ko._f64(q[b, h, r]))
            lse[i] = s.max() + math.log(np.exp(s - s.max()).sum())
            p[i, :e] = np.exp(s - lse[i])
            out[i] = p[i, :e] @ ko._f64(v[b, g])[:e]
        return out, lse, p
    check([ta.test_dense_prefill_matches_causal_library_sdpa], dense_prefill_rows=dense_prefill_rows)


def test_tile_pool_over_one_head_is_caught():
    def tile_pool_one(q, k, b, t, g, tile=128, scale=None):
        q = np.asarray(q)
        Hq, N = q.shape[1], q.shape[2]
        G = Hq // np.asarray(k).shape[1]
        lo, hi = tile * t, min(N, tile * (t + 1))
        _, _, p = ko.dense_prefill_rows(q, k, k, b, g * G, range(lo, hi), scale)  # planted: one head
        return p[:, :hi].sum(axis=0)
    check([ta.test_tile_pool_matches_library_probabilities], tile_pool_one=tile_pool_one)


def test_tile_prefix_off_by_one_tile_is_caught():
    def prefill_tile_k(t, n, tile=128, pct=10, round_to=64, k_min=256):
        p = min(n, tile * t)                                                # planted: P_t = 128 t
        return p, ko.topk_for_len(p, pct, round_to, k_min)
    check([ta.test_anchor_prefill_tiles_zero_and_one_are_dense, tt.test_k_rule_golden],
          prefill_tile_k=prefill_tile_k)


# ---------------------------------------------------------------------------
# Top-k and the k rule
# ---------------------------------------------------------------------------

def test_ties_to_higher_index_are_caught():
    def topk_full_sort(scores, k):
        s = np.asarray(scores, dtype=np.float64).reshape(-1)
        n = s.shape[0]
        k = int(min(max(k, 0), n))
        order = np.lexsort((-np.arange(n), -s))                              # planted: ties high
        return np.sort(order[:k]).astype(np.int64)
    check([tt.test_topk_brute_force_tiny, tt.test_topk_constant_row_and_k_ge_n],
          topk_full_sort=topk_full_sort)


def test_smallest_instead_of_largest_is_caught():
    def topk_full_sort(scores, k):
        s = np.asarray(scores, dtype=np.float64).reshape(-1)
        n = s.shape[0]
        k = int(min(max(k, 0), n))
        order = np.lexsort((np.arange(n), s))                                # planted: sign
        return np.sort(order[:k]).astype(np.int64)
    check([tt.test_topk_brute_force_tiny, tt.test_topk_matches_stable_argsort],
          topk_full_sort=topk_full_sort)


def test_k_rounded_down_is_caught():
    def topk_for_len(n, pct=10, round_to=64, k_min=128):
        tenth = round_to * ((n * pct) // (100 * round_to))                   # planted: floor
        return int(min(n, max(k_min, tenth)))
    check([tt.test_k_rule_golden, tt.test_k_rule_is_nearest_multiple_of_64], topk_for_len=topk_for_len)


def test_k_minimum_dropped_is_caught():
    def topk_for_len(n, pct=10, round_to=64, k_min=128):
        return int(min(n, round_to * ((n * pct + 50 * round_to) // (100 * round_to))))  # planted
    check([tt.test_k_rule_golden], topk_for_len=topk_for_len)


# ---------------------------------------------------------------------------
# calibration: eq. sim, eq. w, head maps, the DP
# ---------------------------------------------------------------------------

def test_sim_over_total_mass_is_caught():
    def sim(p_a, p_b, k):
        p_a, p_b = ko._f64(p_a).reshape(-1), ko._f64(p_b).reshape(-1)
        return float(p_b[ko.topk_full_sort(p_a, k)].sum() / p_b.sum())      # planted: denominator
    check([tc.test_sim_self_is_one_and_bounded, tc.test_sim_denominator_is_best_k_subset_mass,
           tc.test_sim_closed_form_small], sim=sim)


def test_sim_with_swapped_layers_is_caught():
    def sim(p_a, p_b, k):
        return ORIG["sim"](p_b, p_a, k)                                     # planted: a and b swapped
    check([tc.test_sim_closed_form_small, tc.test_sim_denominator_is_best_k_subset_mass], sim=sim)


def test_layer_weight_without_one_minus_is_caught():
    def layer_weight(x, y):
        return 1.0 - ORIG["layer_weight"](x, y)                              # planted: mean cosine
    check([tc.test_layer_weight_closed_forms], layer_weight=layer_weight)


def test_head_map_ties_to_higher_head_are_caught():
    def head_map_from_similarity(M):
        M = ko._f64(M)
        return np.array([max(range(M.shape[0]), key=lambda ga: (M[ga, gb], ga))  # planted: ties high
                         for gb in range(M.shape[1])], dtype=np.int32)
    check([tc.test_head_map_ties_go_to_lower_head], head_map_from_similarity=head_map_from_similarity)


def test_transposed_head_similarity_is_caught():
    def head_similarity(pooled_a, pooled_b, k):
        return ORIG["head_similarity"](pooled_a, pooled_b, k).T              # planted: transposed
    check([tc.test_head_similarity_permuted_heads, tc.test_head_similarity_matches_definition_by_brute_force],
          head_similarity=head_similarity)


def test_greedy_anchor_choice_is_caught():
    def dp_select_anchors(S, M):
        S = ko._f64(S)
        L = S.shape[0]
        # planted: layer 0 plus the M - 1 layers with the largest own similarity row sums
        rest = sorted(range(1, L), key=lambda i: -S[i, i:].sum())[: M - 1]
        anchors = sorted([0] + rest)
        return anchors, ko.coverage_score(S, anchors)
    check([tc.test_dp_matches_brute_force], dp_select_anchors=dp_select_anchors)


def test_dp_segment_served_by_next_anchor_is_caught():
    def coverage_score(S, anchors):
        S = ko._f64(S)
        L = S.shape[0]
        nxt = lambda l: min([a for a in anchors if a >= l], default=anchors[-1])  # planted: next anchor
        return float(sum(S[nxt(l), l] for l in range(L)))
    check([tc.test_dp_matches_brute_force], coverage_score=coverage_score)


# ---------------------------------------------------------------------------
# tile Top-k and the decode layer stack
# ---------------------------------------------------------------------------

def _tile_topk_variant(k_of_tile=None, pad=-1, kmax_tile=None):
    """tile_topk with one step changed (the rest as in the oracle)."""
    def tile_topk(pooled_rows, n, tile=128, pct=10, round_to=64, k_min=256):
        B, T, Hkv = len(pooled_rows), len(pooled_rows[0]), len(pooled_rows[0][0])
        kt = (lambda t: ko.prefill_tile_k(t, n, tile, pct, round_to, k_min)[1])
        k_max = kt(T - 1 if kmax_tile is None else kmax_tile(T))
        idx = np.full((B, T, Hkv, k_max), pad, dtype=np.int64)
        for b in range(B):
            for t in range(T):
                k_t = min(kt(t if k_of_tile is None else k_of_tile(t)), k_max)
                for g in range(Hkv):
                    idx[b, t, g, :k_t] = ko.topk_full_sort(pooled_rows[b][t][g], k_t)
        return idx
    return tile_topk


TILE_PINS = [tt.test_tile_topk_brute_force_per_tile_k_and_padding,
             tt.test_tile_topk_k_max_comes_from_the_last_tile]


def test_tile_topk_with_next_tiles_k_is_caught():
    check(TILE_PINS, tile_topk=_tile_topk_variant(k_of_tile=lambda t: t + 1))   # planted: k_{t+1}


def test_tile_topk_without_minus_one_padding_is_caught():
    check(TILE_PINS, tile_topk=_tile_topk_variant(pad=0))                       # planted: 0 padding


def test_tile_topk_k_max_from_first_tile_is_caught():
    check(TILE_PINS, tile_topk=_tile_topk_variant(kmax_tile=lambda T: 0))       # planted: k_max = k_0


def _stack_variant(anchor_rule=None, own_map=False, anchor_values=False):
    """run_decode_layerstack with one step changed."""
    def run_decode_layerstack(layers, anchors, head_maps, topk, scale=None):
        outs, idx_by_anchor = [], {}
        for l, lay in enumerate(layers):
            if l in anchors:
                out, _, _, idx = ko.anchor_decode(lay["q"], lay["k"], lay["v"], topk, scale)
                idx_by_anchor[l] = idx
            else:
                a = ko.anchor_of(l, anchors) if anchor_rule is None else anchor_rule(l, anchors)
                hm = list(range(len(head_maps[l]))) if own_map else head_maps[l]
                v = layers[a]["v"] if anchor_values else lay["v"]
                out = ko.reuse_decode(lay["q"], lay["k"], v, idx_by_anchor[a], hm, scale)
            outs.append(out)
        return outs, idx_by_anchor
    return run_decode_layerstack


STACK_PINS = [ta.test_layer_stack_with_one_selected_key_is_closed_form,
              ta.test_layer_stack_with_full_lists_is_dense_everywhere]


def test_layer_stack_reusing_the_first_anchor_is_caught():
    check(STACK_PINS, run_decode_layerstack=_stack_variant(anchor_rule=lambda l, A: A[0]))


def test_layer_stack_ignoring_the_head_map_is_caught():
    check(STACK_PINS, run_decode_layerstack=_stack_variant(own_map=True))


def test_layer_stack_with_the_anchors_values_is_caught():
    check(STACK_PINS, run_decode_layerstack=_stack_variant(anchor_values=True))


LAYER_PINS = [ta.test_anchor_and_reuse_prefill_layers_against_library_routines]
DECODE_LAYER_PINS = [ta.test_anchor_and_reuse_decode_layers_against_library_routines]


def _anchor_prefill_variant(rule_ignored=False, pool_tile=None):
    """anchor_prefill with one step changed."""
    def anchor_prefill(q, k, v, tile=128, pct=10, round_to=64, k_min=256, scale=None):
        out, lse = ko.dense_prefill(q, k, v, scale)
        pooled = ko.tile_pool(q, k, pool_tile or tile, scale)
        if rule_ignored:
            pct, round_to, k_min = 10, 64, 256
        return out, lse, pooled, ko.tile_topk(pooled, np.asarray(q).shape[2], tile, pct, round_to, k_min)
    return anchor_prefill


def test_anchor_prefill_ignoring_the_rule_is_caught():
    check(LAYER_PINS, anchor_prefill=_anchor_prefill_variant(rule_ignored=True))


def test_anchor_prefill_pooling_single_rows_is_caught():
    check(LAYER_PINS, anchor_prefill=_anchor_prefill_variant(pool_tile=1))


def test_reuse_prefill_ignoring_the_head_map_is_caught():
    check(LAYER_PINS, reuse_prefill=lambda q, k, v, idx, head_map, tile=128, scale=None:
          ko.sparse_prefill(q, k, v, idx, None, tile, scale))


def test_reuse_decode_ignoring_the_head_map_is_caught():
    check(DECODE_LAYER_PINS, reuse_decode=lambda q, k, v, idx, head_map, scale=None:
          ko.sparse_decode(q, k, v, idx, None, scale)[0])


def test_every_planted_mistake_is_restored():
    for name, fn in ORIG.items():
        assert getattr(ko, name) is fn
    for name in oracle.__all__:
        assert getattr(oracle, name) is ORIG[name]

"""Pins of the oracle's router (logits, sigmoid scores, biased top-k,
renormalisation) and permutation, against closed forms, fp64 bounds and
numpy's stable sorts."""
import json
import os

import numpy as np
import pytest

import oracle
from int4_routed_expert_moe_amd import synthetic
from tests import refmath

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_router(T, H, E, seed, w_std=0.02):
    g = np.random.default_rng(seed)
    x = refmath.bf16_from_f32(g.standard_normal((T, H)).astype(np.float32))
    w = refmath.bf16_from_f32((g.standard_normal((E, H)) * w_std).astype(np.float32))
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    return x, w, b


def test_one_hot_logits_are_router_weights():
    H, E = 256, 16
    _, w, _ = _rand_router(1, H, E, 0)
    cols = np.array([0, 1, 31, 32, 33, 100, 255])
    x = np.zeros((len(cols), H), np.uint16)
    x[np.arange(len(cols)), cols] = 0x3F80  # bf16 1.0
    l = oracle.router_logits(x, w)
    np.testing.assert_array_equal(l, refmath.bf16_to_f32(w[:, cols]).T)


def test_logits_within_two_level_fp32_bound():
    """Blocks of 64 summed in order, then the H/64 block sums in order: the
    rounding error is at most gamma_(64 + H/64) times the sum of |products|."""
    T, H, E = 6, 7168, 24
    x, w, _ = _rand_router(T, H, E, 1)
    l = oracle.router_logits(x, w).astype(np.float64)
    xf = refmath.bf16_to_f32(x).astype(np.float64)
    wf = refmath.bf16_to_f32(w).astype(np.float64)
    exact = xf @ wf.T
    u = 2.0 ** -24
    n = 64 + H // 64
    gamma = n * u / (1 - n * u)
    bound = gamma * (np.abs(xf) @ np.abs(wf).T)
    assert np.all(np.abs(l - exact) <= bound)


def test_selection_is_stable_sort_of_biased_scores():
    T, H, E, k = 64, 256, 16, 4
    x, w, b = _rand_router(T, H, E, 2)
    idx, wt, logits, scores = oracle.route(x, w, b, k, True, return_scores=True)
    np.testing.assert_array_equal(scores, oracle.sigmoid_ref_n(logits).reshape(T, E))
    c = scores + b  # fp32 add, the ranking key
    ref = np.argsort(-c, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref)


def test_ties_pick_lower_expert_index():
    T, H, E, k = 8, 64, 12, 5
    x, w, _ = _rand_router(T, H, E, 3)
    # experts 2,3,4 share one router row, 7 and 9 share another; equal biases
    w[3] = w[2]
    w[4] = w[2]
    w[9] = w[7]
    b = np.zeros(E, np.float32)
    idx, _ = oracle.route(x, w, b, k, True)
    for t in range(T):
        sel = list(idx[t])
        for grp in ([2, 3, 4], [7, 9]):
            pos = [sel.index(e) for e in grp if e in sel]
            chosen = [e for e in grp if e in sel]
            # members of a tie group appear in ascending order and as a prefix of the group
            assert chosen == grp[:len(chosen)]
            assert pos == sorted(pos)


def test_zero_bias_selects_top_logits():
    T, H, E, k = 64, 256, 16, 3
    x, w, _ = _rand_router(T, H, E, 4)
    idx, _, logits, scores = oracle.route(x, w, np.zeros(E, np.float32), k, True, return_scores=True)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    for t in range(T):
        if len(np.unique(scores[t])) == E:  # no equal scores from distinct logits
            np.testing.assert_array_equal(idx[t], ref[t])


def test_renormalised_weights():
    eps = json.load(open(os.path.join(GOLD, "router_renorm_eps.json")))["eps"]
    T, H, E, k = 64, 256, 16, 4
    x, w, b = _rand_router(T, H, E, 5)
    idx, wt, _, scores = oracle.route(x, w, b, k, True, return_scores=True)
    sel = np.take_along_axis(scores, idx, axis=1).astype(np.float64)
    exact = sel / (sel.sum(axis=1, keepdims=True) + eps)
    assert np.all(np.abs(wt - exact) <= 4 * 2.0 ** -24 * np.abs(exact))
    assert np.all(np.abs(wt.astype(np.float64).sum(axis=1) - 1.0) <= k * 2.0 ** -23)
    idx2, wt2 = oracle.route(x, w, b, k, False)
    np.testing.assert_array_equal(idx2, idx)
    np.testing.assert_array_equal(wt2, np.take_along_axis(scores, idx, axis=1))


def test_k_equals_e_selects_every_expert_once():
    T, H, E = 16, 64, 8
    x, w, b = _rand_router(T, H, E, 6)
    idx, _ = oracle.route(x, w, b, E, True)
    for t in range(T):
        assert sorted(idx[t]) == list(range(E))


@pytest.mark.parametrize("T,k,E,seed", [(64, 2, 16, 0), (64, 8, 384, 1), (8192, 8, 384, 2), (1, 1, 1, 3)])
def test_permute_is_stable_counting_sort(T, k, E, seed):
    g = np.random.default_rng(seed)
    idx = g.integers(0, E, (T, k)).astype(np.int32)
    if E > 4:
        idx[idx == 3] = 4  # force an empty expert
    counts, offsets, sorted_slot, slot_pos = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(counts, np.bincount(flat, minlength=E))
    assert counts.sum() == T * k
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    np.testing.assert_array_equal(sorted_slot, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(slot_pos[sorted_slot], np.arange(T * k))
    np.testing.assert_array_equal(sorted_slot[slot_pos], np.arange(T * k))


def test_permute_single_expert():
    idx = np.full((10, 3), 5, np.int32)
    counts, offsets, ss, sp = oracle.permute(idx, 8)
    assert counts[5] == 30 and counts.sum() == 30
    np.testing.assert_array_equal(ss, np.arange(30))
    np.testing.assert_array_equal(offsets[6:], 30)


def test_tiny_config_routing_invariants():
    inp = synthetic.make_inputs(1, with_experts=False)
    cfg = inp["cfg"]
    idx, wt = oracle.route(inp["x"], inp["router_w"], inp["router_b"], cfg["k"], True)
    assert idx.shape == (cfg["T"], cfg["k"])
    assert np.all((idx >= 0) & (idx < cfg["E"]))
    for t in range(cfg["T"]):
        assert len(set(idx[t])) == cfg["k"]
    assert np.all(wt > 0)


def test_zipf_fixture_routing_on_exact_workload():
    """The calibrated bias gives 77 dead experts with zero tokens and a heavy head."""
    bias = synthetic.load_bias_file(os.path.join(GOLD, "zipf_bias_k25.txt"))
    inp = synthetic.make_inputs(4, router_bias=bias, with_experts=False)
    cfg = inp["cfg"]
    idx, _ = oracle.route(inp["x"], inp["router_w"], bias, cfg["k"], True)
    counts = np.bincount(idx.ravel(), minlength=cfg["E"])
    dead = bias == np.float32(-4.0)
    assert dead.sum() == round(0.2 * cfg["E"])
    assert counts[dead].sum() == 0
    assert counts.sum() == cfg["T"] * cfg["k"]
    assert counts.max() > cfg["T"] // 2


# ---------------------------------------------------------------- group-limited selection
# ("Kimi K2.5 donor reference", MoEGate.forward records: group scores, group idx,
# score mask, topk idx; readings in oracle_topk_grouped_from_scores)

def _scores(g, T, E):
    s = g.uniform(0.01, 0.99, (T, E)).astype(np.float32)
    b = g.uniform(-0.1, 0.1, E).astype(np.float32)
    return s, b


@pytest.mark.parametrize("E,n_group,k", [(16, 4, 3), (384, 8, 8)])
def test_grouped_with_every_group_kept_is_plain_routing(E, n_group, k):
    g = np.random.default_rng(11)
    s, b = _scores(g, 40, E)
    idx0, w0 = oracle.topk_from_scores(s, b, k)
    for ng, tg in ((1, 1), (n_group, n_group)):
        idx, w = oracle.topk_grouped_from_scores(s, b, k, ng, tg)
        np.testing.assert_array_equal(idx, idx0)
        np.testing.assert_array_equal(w, w0)


@pytest.mark.parametrize("E,n_group,topk_group,k,seed", [(64, 8, 3, 6, 0), (384, 8, 4, 8, 1), (48, 4, 1, 5, 2)])
def test_grouped_selection_is_sort_of_masked_scores(E, n_group, topk_group, k, seed):
    """Group scores from a library sort of each group (two largest, added in fp32),
    kept groups and experts from stable sorts with the index as tie-breaker."""
    g = np.random.default_rng(seed)
    T = 50
    s, b = _scores(g, T, E)
    idx, _ = oracle.topk_grouped_from_scores(s, b, k, n_group, topk_group)
    c = (s + b).astype(np.float32)
    G = E // n_group
    top2 = np.sort(c.reshape(T, n_group, G), axis=2)[:, :, ::-1][:, :, :2]
    gs = (top2[:, :, 0] + top2[:, :, 1]).astype(np.float32)
    for t in range(T):
        keep = np.lexsort((np.arange(n_group), -gs[t]))[:topk_group]
        allowed = np.isin(np.arange(E) // G, keep)
        cand = np.nonzero(allowed)[0]
        order = cand[np.lexsort((cand, -c[t, cand]))][:k]
        np.testing.assert_array_equal(idx[t], order)


def test_grouped_worked_example():
    """Eight experts in four groups of two.  Biased scores
    c = [0.9, 0.1 | 0.5, 0.5 | 0.8, 0.0 | 0.3, 0.3] give group scores
    [1.0, 1.0, 0.8, 0.6]; keeping two groups keeps 0 and 1, so the top two are
    experts 0 and 2 (2 before its tie 3), where ungrouped routing picks 0 and 4."""
    c = np.array([[0.9, 0.1, 0.5, 0.5, 0.8, 0.0, 0.3, 0.3]], dtype=np.float32)
    s = c.copy()
    b = np.zeros(8, dtype=np.float32)
    idx, w = oracle.topk_grouped_from_scores(s, b, 2, 4, 2)
    np.testing.assert_array_equal(idx, [[0, 2]])
    idx_plain, _ = oracle.topk_from_scores(s, b, 2)
    np.testing.assert_array_equal(idx_plain, [[0, 4]])
    d = np.float32(np.float32(0.9) + np.float32(0.5)) + np.float32(1e-20)
    np.testing.assert_array_equal(w, [[np.float32(0.9) / d, np.float32(0.5) / d]])


def test_grouped_tied_groups_keep_lower_index():
    """Groups 1 and 3 tie on their score; with one group kept, group 1 wins."""
    c = np.array([[0.1, 0.2, 0.6, 0.3, 0.2, 0.1, 0.3, 0.6]], dtype=np.float32)
    idx, _ = oracle.topk_grouped_from_scores(c, np.zeros(8, np.float32), 2, 4, 1)
    np.testing.assert_array_equal(idx, [[2, 3]])


def test_grouped_scaling_factor_multiplies_weights():
    g = np.random.default_rng(5)
    s, b = _scores(g, 30, 64)
    _, w1 = oracle.topk_grouped_from_scores(s, b, 6, 8, 3, True, 1.0)
    _, w25 = oracle.topk_grouped_from_scores(s, b, 6, 8, 3, True, 2.5)
    np.testing.assert_array_equal(w25, (w1 * np.float32(2.5)).astype(np.float32))
    assert np.all(np.abs(w1.sum(axis=1) - 1.0) <= 6 * 2.0 ** -24 * 4)

"""Pins of the routing oracle against what the pages and mathematics fix."""

import itertools
import json
import os

import numpy as np
import pytest

import oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Worked example of the GroupedTopK page, section 四.

def test_gtk_worked_example_softmax(golden_dir):
    g = _load(golden_dir, "gtk_worked_example.json")
    s = np.array(g["scores"])
    # softmax(log s) = s / sum(s): same order as the page's scores.
    logits = np.log(s)
    w, ids = oracle.grouped_topk(logits[None], g["topk"], True,
                                 g["num_expert_group"], g["topk_group"])
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_allclose(w[0], [0.9 / 1.7, 0.8 / 1.7], rtol=0, atol=1e-15)


def test_gtk_worked_example_sigmoid(golden_dir):
    g = _load(golden_dir, "gtk_worked_example.json")
    s = np.array(g["scores"])
    logits = np.log(s / (1.0 - s))          # sigmoid(logit(s)) = s
    w, ids = oracle.grouped_topk(logits[None], g["topk"], False,
                                 g["num_expert_group"], g["topk_group"],
                                 scoring="sigmoid", routed_scaling_factor=1.0)
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_allclose(w[0], [0.9, 0.8], atol=1e-15)


def test_gtk_worked_example_masked_row(golden_dir):
    """With topk=4 the picks must follow the page's masked score row
    (experts of dropped groups are -inf): .9 (4), .8 (1), .7 (5), .1 (0)."""
    g = _load(golden_dir, "gtk_worked_example.json")
    masked = g["masked_scores"]
    expect = [i for i in sorted(range(8), key=lambda i: -(masked[i] or -1.0))
              if masked[i] is not None][:4]
    assert expect == [4, 1, 5, 0]
    w, ids = oracle.grouped_topk(np.log(np.array(g["scores"]))[None], 4, True,
                                 g["num_expert_group"], g["topk_group"])
    assert ids[0].tolist() == expect
    # every pick lies in a kept group
    kept = set(g["kept_groups"])
    assert all(i // 2 in kept for i in ids[0])


def test_gtk_group_maxima_not_top2_sum():
    """Group score is the in-group MAX ([GTK] §3.2).  Group 0 = {.5, .5}
    (top-2 sum 1.0) against group 1 = {.6, .0} (sum .6): the max rule keeps
    group 1, a top-2-sum rule would keep group 0."""
    s = np.array([0.5, 0.5, 0.6, 0.0001])
    w, ids = oracle.grouped_topk(np.log(s)[None], 1, True, 2, 1)
    assert ids[0].tolist() == [2]


# ---------------------------------------------------------------------------
# Seeded printout of the mini-sglang page.

def test_msg_seeded_routing(golden_dir):
    torch = pytest.importorskip("torch")
    g = _load(golden_dir, "msg_seeded_example.json")
    torch.manual_seed(0)
    _x, gating = torch.randn(g["T"], g["H"]), torch.randn(g["T"], g["E"])
    logits = gating.double().numpy()
    w, ids = oracle.select_experts(logits, g["topk"], g["renormalize"])
    assert ids.tolist() == g["ids"]
    np.testing.assert_allclose(np.round(w, 3), g["weights_3dp"], atol=1e-12)
    # the grouped form with one group is the same routing
    w2, ids2 = oracle.grouped_topk(logits, g["topk"], True, 1, 1)
    assert ids2.tolist() == g["ids"]
    np.testing.assert_allclose(w2, w, atol=1e-15)


# ---------------------------------------------------------------------------
# Brute force on tiny inputs: rank-count definition of a sorted top-k with
# lower-index tie-break, at expert level and at group level.

def _rank_count_topk(values, k):
    n = len(values)
    pos = {}
    for e in range(n):
        if values[e] == -np.inf:
            continue
        r = sum(1 for j in range(n)
                if values[j] > values[e] or (values[j] == values[e] and j < e))
        if r < k:
            pos[r] = e
    return [pos[r] for r in range(k)]


def _brute_grouped(scores, k, G, Kg):
    E = len(scores)
    P = E // G
    gs = [max(scores[i * P:(i + 1) * P]) for i in range(G)]
    kept = _rank_count_topk(gs, Kg)
    masked = [scores[e] if (e // P) in kept else -np.inf for e in range(E)]
    return _rank_count_topk(masked, k), kept


@pytest.mark.parametrize("seed", range(40))
def test_bruteforce_tiny(seed):
    rng = np.random.default_rng(1000 + seed)
    G = int(rng.choice([1, 2, 4]))
    P = int(rng.choice([1, 2, 3]))
    E = G * P
    Kg = int(rng.integers(1, G + 1))
    k = int(rng.integers(1, Kg * P + 1))
    # few distinct values -> many exact ties, on purpose
    logits = rng.integers(-2, 3, size=(3, E)).astype(np.float64) * 0.5
    for scoring in ("softmax", "sigmoid"):
        w, ids = oracle.grouped_topk(logits, k, True, G, Kg, scoring)
        s = (oracle.softmax_scores(logits) if scoring == "softmax"
             else oracle.sigmoid_scores(logits))
        for t in range(logits.shape[0]):
            expect, _ = _brute_grouped(list(s[t]), k, G, Kg)
            assert ids[t].tolist() == expect


def test_all_equal_logits_pick_lowest_ids():
    w, ids = oracle.grouped_topk(np.zeros((2, 16)), 3, True, 4, 2)
    # groups tie -> groups 0,1 kept; experts tie -> 0,1,2
    assert ids.tolist() == [[0, 1, 2], [0, 1, 2]]
    np.testing.assert_allclose(w, 1.0 / 3.0, atol=1e-15)


def test_ties_inside_group():
    logits = np.array([[0.0, 3.0, 3.0, 1.0, 3.0, 0.0, 0.0, 0.0]])
    _, ids = oracle.grouped_topk(logits, 3, True, 2, 1)
    assert ids[0].tolist() == [1, 2, 3]        # group 0 kept (tie -> lower)


# ---------------------------------------------------------------------------
# Closed forms and special cases.

def test_topk_equals_E_is_sorted_softmax():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 12))
    w, ids = oracle.grouped_topk(x, 12, False, 1, 1)
    p = np.exp(x - x.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(w, -np.sort(-p, axis=1), atol=1e-15)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)


def test_top1_renormalised_is_scale():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 32))
    w, ids = oracle.grouped_topk(x, 1, True, 4, 2, routed_scaling_factor=2.5)
    np.testing.assert_allclose(w, 2.5, atol=1e-15)
    assert (ids[:, 0] == np.argmax(x, axis=1)).all()


def test_renormalised_softmax_shortcut():
    """[GTK] §七: with renormalize the full denominator cancels, so the
    weights are a softmax over the selected logits alone."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 64))
    w, ids = oracle.grouped_topk(x, 8, True, 8, 4)
    sel = np.take_along_axis(x, ids, 1)
    e = np.exp(sel - sel.max(1, keepdims=True))
    np.testing.assert_allclose(w, e / e.sum(1, keepdims=True), atol=1e-14)


def test_unrenormalised_keeps_full_denominator():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((3, 16))
    w, ids = oracle.grouped_topk(x, 4, False, 4, 2, routed_scaling_factor=3.0)
    full = np.exp(x) / np.exp(x).sum(1, keepdims=True)
    np.testing.assert_allclose(w, 3.0 * np.take_along_axis(full, ids, 1),
                               atol=1e-14)


def test_invariants_routing_config():
    """[GTK] §九 invariants at the routing workload's shape."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((83, 256)).astype(np.float32)
    for scale in (1.0, 2.5):
        w, ids = oracle.grouped_topk(x, 8, True, 8, 4, routed_scaling_factor=scale)
        assert ids.shape == (83, 8)
        assert ((ids >= 0) & (ids < 256)).all()
        for t in range(83):
            assert len(set(ids[t])) == 8
            groups = set(int(i) // 32 for i in ids[t])
            assert len(groups) <= 4
            # kept groups are exactly the 4 with the largest in-group max
            gmax = x[t].reshape(8, 32).max(1)
            kept = set(np.argsort(-gmax, kind="stable")[:4].tolist())
            assert groups <= kept
        np.testing.assert_allclose(w.sum(1), scale, rtol=1e-14)
        assert (np.diff(w, axis=1) <= 0).all()      # descending weights


def test_rows_independent():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((10, 32))
    perm = rng.permutation(10)
    w, ids = oracle.grouped_topk(x, 4, True, 4, 2)
    wp, idsp = oracle.grouped_topk(x[perm], 4, True, 4, 2)
    assert (idsp == ids[perm]).all()
    np.testing.assert_array_equal(wp, w[perm])


def test_neg_inf_logits_rank_last():
    x = np.array([[-np.inf, 0.5, -np.inf, 0.1]])
    w, ids = oracle.grouped_topk(x, 3, True, 1, 1)
    assert ids[0].tolist() == [1, 3, 0]
    assert w[0, 2] == 0.0


@pytest.mark.parametrize("bad", [dict(num_expert_group=3),
                                 dict(topk_group=5),
                                 dict(topk=9, topk_group=1)])
def test_bad_configs_raise(bad):
    args = dict(topk=2, renormalize=True, num_expert_group=4, topk_group=2)
    args.update(bad)
    with pytest.raises(ValueError):
        oracle.grouped_topk(np.zeros((1, 32)), **args)

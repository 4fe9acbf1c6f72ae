"""Comparison rules between the HIP path and the oracle.

* integer outputs (ids, alignment metadata): bit-exact;
* routing: a position may differ only where the oracle's scores of the two
  ids differ by less than 1e-6 (and likewise for the group maxima), and the
  GPU's selection must itself be a valid top-k within that slack; accepted
  positions are re-scored by the oracle for the weight check;
* floating outputs: err = max|y - r| / max|r| against a stated bar.
"""

import numpy as np

import oracle

TIE_SLACK = 1e-6
BAR_ROUTING_W = 1e-5
BAR_BF16 = 2e-2
BAR_INT8 = 3e-2


def max_abs_rel(y, r):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    denom = np.max(np.abs(r)) if r.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(y - r))) if r.size else 0.0
    return float(np.max(np.abs(y - r)) / denom)


def _scores(logits, scoring):
    return (oracle.softmax_scores(logits) if scoring == "softmax"
            else oracle.sigmoid_scores(logits))


def check_routing(gpu_w, gpu_ids, logits, topk, renormalize, G, Kg, scoring, scale,
                  w_bar=BAR_ROUTING_W):
    """Returns (n_exact_rows, n_near_tie_rows, weight_err).  Raises
    AssertionError on any mismatch outside the near-tie rule."""
    logits = np.asarray(logits, dtype=np.float64)
    gpu_ids = np.asarray(gpu_ids).astype(np.int64)
    gpu_w = np.asarray(gpu_w, dtype=np.float64)
    w_ref, ids_ref = oracle.grouped_topk(logits, topk, renormalize, G, Kg, scoring, scale)
    s = _scores(logits, scoring)
    T, E = logits.shape
    P = E // G
    exact = ties = 0
    w_expect = w_ref.copy()
    for t in range(T):
        if (gpu_ids[t] == ids_ref[t]).all():
            exact += 1
            continue
        g = gpu_ids[t]
        assert len(set(g.tolist())) == topk, "token %d: repeated ids %s" % (t, g)
        assert ((g >= 0) & (g < E)).all(), "token %d: id out of range" % t
        gaps = np.abs(s[t, g] - s[t, ids_ref[t]])
        assert (gaps < TIE_SLACK).all(), \
            "token %d: ids %s vs oracle %s (score gaps %s)" % (t, g, ids_ref[t], gaps)
        gs = s[t].reshape(G, P).max(axis=1)
        kth = np.sort(gs)[::-1][Kg - 1]
        for gi in set((g // P).tolist()):
            assert gs[gi] >= kth - TIE_SLACK, "token %d: group %d not a valid pick" % (t, gi)
        # descending within slack
        assert (np.diff(s[t, g]) <= TIE_SLACK).all()
        ws = s[t, g].copy()
        if renormalize:
            ws = ws / ws.sum()
        w_expect[t] = ws * scale
        ties += 1
    err = max_abs_rel(gpu_w, w_expect)
    assert err <= w_bar, "routing weight error %.3g > %.3g" % (err, w_bar)
    return exact, ties, err

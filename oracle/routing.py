"""Oracle: routing scores, grouped top-k and plain top-k (test infrastructure).

Test infrastructure only (see ``oracle/__init__.py``).  float64 throughout.

Readings where the pages leave a step open:
* ties (equal scores, equal group scores) go to the LOWER index; [GTK] §八
  only raises the question;
* the K ids come out in descending score order, ties by ascending index
  (the order a sorted top-k gives, [GTK] §八 last question);
* routed_scaling_factor multiplies the weights whether or not they were
  renormalised ([GTK] §3.6 states it as the last step);
* softmax with renormalize=False keeps the full-row denominator ([GTK] §七,
  first limit of the shortcut).
"""

import numpy as np


def softmax_scores(logits):
    """Row softmax with the row max subtracted first ([GTK] §3.1, softmax)."""
    x = np.asarray(logits, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def sigmoid_scores(logits):
    """Independent per-expert score 1/(1+exp(-x)) ([GTK] §3.1, sigmoid)."""
    x = np.asarray(logits, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def _top_indices(values, k):
    """Indices of the k largest values, largest first, equal values by
    ascending index.  A stable sort of the negated values gives exactly that
    order; -inf entries sort last."""
    order = np.argsort(-values, kind="stable")
    return order[:k]


def grouped_topk(logits, topk, renormalize=True, num_expert_group=1,
                 topk_group=1, scoring="softmax", routed_scaling_factor=1.0):
    """GroupedTopK routing, the steps of [GTK] §3.1-§3.6 in the page's order.

    logits: [T, E] router logits (the gating_output of [GTK] §二).
    Returns (topk_weights float64 [T, topk], topk_ids int64 [T, topk]).

    1. scores s = softmax or sigmoid of the logits           (§3.1)
    2. group score g_i = max of s over group i's experts      (§3.2)
    3. keep the topk_group groups with the largest g          (§3.3)
    4. experts outside the kept groups get score -inf         (§3.4)
    5. ids = top-k of the masked scores, w = their scores     (§3.5)
    6. if renormalize: w <- w / sum(w)                        (§3.6)
    7. w <- w * routed_scaling_factor                         (§3.6)
    """
    x = np.asarray(logits, dtype=np.float64)
    T, E = x.shape
    G = int(num_expert_group)
    if G < 1 or E % G != 0:
        raise ValueError("E must be divisible by num_expert_group")
    P = E // G
    if not (1 <= topk_group <= G):
        raise ValueError("topk_group out of range")
    if not (1 <= topk <= topk_group * P):
        raise ValueError("topk exceeds the candidate experts")
    if scoring == "softmax":
        s = softmax_scores(x)
    elif scoring == "sigmoid":
        s = sigmoid_scores(x)
    else:
        raise ValueError("scoring must be softmax or sigmoid")

    weights = np.zeros((T, topk), dtype=np.float64)
    ids = np.zeros((T, topk), dtype=np.int64)
    for t in range(T):
        row = s[t]
        group_scores = np.array([np.max(row[i * P:(i + 1) * P]) for i in range(G)])
        kept = _top_indices(group_scores, topk_group)
        masked = np.full(E, -np.inf)
        for gi in kept:
            masked[gi * P:(gi + 1) * P] = row[gi * P:(gi + 1) * P]
        sel = _top_indices(masked, topk)
        w = row[sel].copy()
        if renormalize:
            w = w / np.sum(w)
        w = w * float(routed_scaling_factor)
        weights[t] = w
        ids[t] = sel
    return weights, ids


def select_experts(gating_output, topk, renormalize=True):
    """Plain top-k routing of [MSG] "路由" (select_experts): softmax over all
    experts, the k largest probabilities, optionally divided by their sum."""
    p = softmax_scores(gating_output)
    T = p.shape[0]
    ids = np.stack([_top_indices(p[t], topk) for t in range(T)]).astype(np.int64)
    w = np.take_along_axis(p, ids, axis=1)
    if renormalize:
        w = w / np.sum(w, axis=1, keepdims=True)
    return w, ids

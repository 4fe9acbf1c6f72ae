"""Oracle: the whole fused-MoE layer forward (test infrastructure; see
``oracle/__init__.py``).  float64 throughout."""

import numpy as np

from .gemm import silu, silu_and_mul
from .routing import grouped_topk


def moe_layer_pair_rows(x, w1, w2, topk_weights, topk_ids):
    """The routing-weighted output of every (token, slot) pair, evaluated one
    expert at a time.

    [MSG] "参考后端" defines the layer output of token t as
        out[t] = sum_k w[t, k] * W2[e] ( silu(W1[e][:I] x_t) * (W1[e][I:] x_t) ),
    e = topk_ids[t, k], and evaluates it per expert.  Here every expert that
    occurs in topk_ids maps the rows of all the (t, k) slots that chose it in
    one matrix product.  x [T, H], w1 [E, 2I, H] (gate rows first),
    w2 [E, H, I].  Returns the terms of that sum, [T, topk, H] float64
    (pair p = t * topk + k is row p of its [T * topk, H] view)."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, dtype=np.float64)
    slots = np.zeros(ids.shape + (x.shape[1],), dtype=np.float64)
    for e in sorted(set(int(v) for v in ids.ravel())):
        tok, slot = np.nonzero(ids == e)            # the slots routed to e
        w1e = np.asarray(w1[e], dtype=np.float64)
        inter = w1e.shape[0] // 2
        act = silu(x[tok] @ w1e[:inter].T) * (x[tok] @ w1e[inter:].T)
        down = act @ np.asarray(w2[e], dtype=np.float64).T
        slots[tok, slot] = wts[tok, slot][:, None] * down
    return slots


def moe_layer_expert_loop(x, w1, w2, topk_weights, topk_ids):
    """The layer output: each token's pair terms (moe_layer_pair_rows,
    computed one expert at a time) summed over its slots.  Returns
    out [T, H] float64."""
    return moe_layer_pair_rows(x, w1, w2, topk_weights, topk_ids).sum(axis=1)


def moe_layer_token_loop(x, w1, w2, topk_weights, topk_ids):
    """The direct per-token, per-expert loop that [MSG] "测试" uses to check
    its reference backend: out[t] = sum_k w[t,k] * W2[e]( silu(g) * u ),
    g = W1[e][:I] x[t], u = W1[e][I:] x[t], e = topk_ids[t, k]."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, dtype=np.float64)
    T, topk = ids.shape
    out = np.zeros((T, x.shape[1]), dtype=np.float64)
    for t in range(T):
        for k in range(topk):
            e = int(ids[t, k])
            w1e = np.asarray(w1[e], dtype=np.float64)
            I = w1e.shape[0] // 2
            g = w1e[:I] @ x[t]
            u = w1e[I:] @ x[t]
            h = (g / (1.0 + np.exp(-g))) * u
            out[t] += wts[t, k] * (np.asarray(w2[e], dtype=np.float64) @ h)
    return out


def dense_swiglu(x, w1e, w2e):
    """One expert applied to every row: silu_and_mul(x @ w1e^T) @ w2e^T.
    With a single expert and weight 1 the layer reduces to this."""
    x = np.asarray(x, dtype=np.float64)
    return silu_and_mul(x @ np.asarray(w1e, dtype=np.float64).T) @ \
        np.asarray(w2e, dtype=np.float64).T


def moe_forward(x, gating, w1, w2, topk, renormalize=True, num_expert_group=1,
                topk_group=1, scoring="softmax", routed_scaling_factor=1.0):
    """[MSG] "fused MoE" (FusedMoeBackend.forward) read as its plain
    definition: route, then the layer.  Routing is [GTK] §3 (plain top-k is
    its G=1 case).  Returns (out [T, H], topk_weights, topk_ids)."""
    w, ids = grouped_topk(gating, topk, renormalize, num_expert_group,
                          topk_group, scoring, routed_scaling_factor)
    return moe_layer_expert_loop(x, w1, w2, w, ids), w, ids

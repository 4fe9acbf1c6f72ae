"""Oracle: the whole fused-MoE layer forward (test infrastructure; see
``oracle/__init__.py``).  float64 throughout."""

import numpy as np

from .gemm import silu_and_mul
from .routing import grouped_topk


def moe_layer_expert_loop(x, w1, w2, topk_weights, topk_ids):
    """[MSG] "参考后端" (TorchMoeBackend): for every expert that some pair
    chose, gather the tokens routed to it, run silu_and_mul(x_t @ w1[e]^T)
    @ w2[e]^T, multiply by the routing weight, and add the rows back into
    their tokens.  x [T, H], w1 [E, 2I, H] (gate rows first), w2 [E, H, I].
    Returns out [T, H] float64."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    T, topk = ids.shape
    flat_ids = ids.reshape(-1)
    token_idx = np.repeat(np.arange(T), topk)
    flat_w = np.asarray(topk_weights, dtype=np.float64).reshape(-1)
    out = np.zeros((T, x.shape[1]), dtype=np.float64)
    for e in np.unique(flat_ids):
        sel = np.flatnonzero(flat_ids == e)
        tokens = token_idx[sel]
        w1e = np.asarray(w1[int(e)], dtype=np.float64)
        w2e = np.asarray(w2[int(e)], dtype=np.float64)
        h = silu_and_mul(x[tokens] @ w1e.T)
        y = (h @ w2e.T) * flat_w[sel][:, None]
        np.add.at(out, tokens, y)
    return out


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

"""Oracle: the fused-MoE layer with INT8 weights and INT8 activations
(test infrastructure; see ``oracle/__init__.py``).

[GMM] §3.2 quantises weights symmetrically per output channel and
activations symmetrically per token, and §5.3 accumulates the integer
products exactly.  [GMM] §4 asks for the activations to be quantised in
the kernel as they are loaded.  Applied to both GEMMs of the [MSG]
reference layer ("参考后端"):
    xq, sx = per-token int8 of x
    gate/up = sx[t] * s1[e, n] * sum_k xq[t, k] * w1q[e, n, k]    (exact sum)
    h = silu(gate) * up
    hq, sh = per-row int8 of h                     (one row per pair)
    y = w[pair] * sh[pair] * s2[e, n] * sum_k hq[k] * w2q[e, n, k]
    out[t] = sum over the token's pairs of y.
The pages fix no precision for the quantisation step.  The kernel takes it
in float32, so the quantiser here does the same (quantize_rows_f32): for
bf16 activations both sides then produce identical codes.  h comes from
float64 arithmetic here and float32 arithmetic in the kernel; a code can
therefore differ by one where h sits on a rounding boundary, a difference
the layer's tolerance covers.  Everything else is float64.
"""

import numpy as np

from .gemm import silu_and_mul


def quantize_rows_f32(x):
    """[GMM] §3.2 symmetric per-row int8 quantisation, in float32:
    scale = max|row| / 127 (float32 division), q = clamp(round(row / scale),
    -127, 127) with the division in float32 and round half to even.  An
    all-zero row gets scale 1 and codes 0 (the pages are silent; same
    reading as quantize_weight_per_channel).  Returns (q int8, scale
    float32)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1, keepdims=True)
    scale = amax / np.float32(127.0)
    scale = np.where(scale == np.float32(0.0), np.float32(1.0), scale).astype(np.float32)
    q = np.clip(np.rint(x / scale), -127, 127).astype(np.int8)
    return q, scale[..., 0]


def _int_dot(aq, bq):
    """Exact integer matrix product of int8 operands (float64 holds every
    partial sum exactly while K * 127^2 < 2^53)."""
    if aq.shape[-1] * 127 * 127 >= 2 ** 53:
        raise ValueError("K too large for an exact float64 integer sum")
    return np.asarray(aq, dtype=np.float64) @ np.asarray(bq, dtype=np.float64).T


def moe_layer_w8a8_expert_loop(x, w1q, s1, w2q, s2, topk_weights, topk_ids):
    """The layer above, evaluated one expert at a time: every expert that
    occurs in topk_ids maps the rows of the (t, k) slots that chose it in one
    exact integer product per GEMM, the scaled slot results are kept in a
    [T, topk, H] array and each token's slots are summed at the end.
    x [T, H] (float values), w1q [E, 2I, H] int8 with s1 [E, 2I],
    w2q [E, H, I] int8 with s2 [E, H], topk_weights / topk_ids [T, topk].
    Returns out [T, H] float64."""
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, dtype=np.float64)
    xq, sx = quantize_rows_f32(x)
    sx = sx.astype(np.float64)
    slots = np.zeros(ids.shape + (np.asarray(x).shape[1],), dtype=np.float64)
    for e in sorted(set(int(v) for v in ids.ravel())):
        tok, slot = np.nonzero(ids == e)            # the slots routed to e
        acc1 = _int_dot(xq[tok], w1q[e])            # exact integer sums
        gate_up = acc1 * sx[tok, None] * np.asarray(s1[e], dtype=np.float64)[None, :]
        hq, sh = quantize_rows_f32(silu_and_mul(gate_up))
        acc2 = _int_dot(hq, w2q[e])
        scale = sh.astype(np.float64)[:, None] * np.asarray(s2[e], dtype=np.float64)[None, :]
        slots[tok, slot] = wts[tok, slot][:, None] * scale * acc2
    return slots.sum(axis=1)


def moe_layer_w8a8_token_loop(x, w1q, s1, w2q, s2, topk_weights, topk_ids):
    """The same layer as a direct loop over tokens and their topk experts
    (an independent formulation used to check the expert loop)."""
    ids = np.asarray(topk_ids)
    wts = np.asarray(topk_weights, dtype=np.float64)
    T, topk = ids.shape
    xq, sx = quantize_rows_f32(x)
    out = np.zeros((T, np.asarray(x).shape[1]), dtype=np.float64)
    for t in range(T):
        xt = xq[t].astype(np.float64)
        for k in range(topk):
            e = int(ids[t, k])
            I = w1q[e].shape[0] // 2
            acc = np.asarray(w1q[e], dtype=np.float64) @ xt
            gu = acc * float(sx[t]) * np.asarray(s1[e], dtype=np.float64)
            g, u = gu[:I], gu[I:]
            h = (g / (1.0 + np.exp(-g))) * u
            hq, sh = quantize_rows_f32(h[None, :])
            acc2 = np.asarray(w2q[e], dtype=np.float64) @ hq[0].astype(np.float64)
            out[t] += wts[t, k] * float(sh[0]) * np.asarray(s2[e], dtype=np.float64) * acc2
    return out

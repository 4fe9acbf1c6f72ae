"""Oracle: the grouped GEMM (GMM) and its INT8 variant (test
infrastructure; see ``oracle/__init__.py``)."""

import numpy as np


def gmm(X, W, expert_offsets):
    """[GMM] §2.1: rows [off[e], off[e+1]) of the expert-sorted input X [M, K]
    form group S_e, and Y[S_e] = X[S_e] @ W[e]^T with W [E, N, K].  Output
    rows stay in input (sorted) order; putting them back into token order is
    the caller's step.  float64."""
    X = np.asarray(X, dtype=np.float64)
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = off.size - 1
    Y = np.zeros((X.shape[0], W.shape[1]), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            Y[lo:hi] = X[lo:hi] @ np.asarray(W[e], dtype=np.float64).T
    return Y


def gmm_int8(Xq, Wq, scales_x, scales_w, expert_offsets):
    """[GMM] §2.1 with the low-precision policy of §2.3 / §3.1 / §5.3:
        Y[m, n] = scales_x[m] * scales_w[e, n] * sum_k Xq[m, k] * Wq[e, n, k]
    for m in [off[e], off[e+1]).  The integer sum is exact: it is formed by a
    float64 matmul of the int8 values, and every product and partial sum is
    an integer of magnitude <= K * 127^2, below 2^53 for any K < 5e11, so no
    step rounds whatever the summation order.  The two scales are applied in
    float64.  Returns float64 [M, N]."""
    K = np.asarray(Xq).shape[1]
    if K * 127 * 127 >= 2 ** 53:
        raise ValueError("K too large for an exact float64 integer sum")
    Xq = np.asarray(Xq, dtype=np.float64)
    sx = np.asarray(scales_x, dtype=np.float64)
    sw = np.asarray(scales_w, dtype=np.float64)
    off = np.asarray(expert_offsets, dtype=np.int64)
    E = off.size - 1
    Y = np.zeros((Xq.shape[0], Wq.shape[1]), dtype=np.float64)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi <= lo:
            continue
        acc = Xq[lo:hi] @ np.asarray(Wq[e], dtype=np.float64).T   # exact integers
        Y[lo:hi] = acc * sx[lo:hi, None] * sw[e][None, :]
    return Y


def quantize_weight_per_channel(w):
    """[GMM] §3.2: symmetric per-output-channel int8.  w [N, K] (or [E, N, K]);
    scale = max|w| over K / 127, q = clamp(round(w / scale), -127, 127) with
    round-half-to-even (the page's torch.round).  An all-zero channel would
    divide by zero; the pages are silent, this reading uses scale 1, q 0."""
    w = np.asarray(w, dtype=np.float64)
    scale = np.max(np.abs(w), axis=-1, keepdims=True) / 127.0
    scale = np.where(scale == 0.0, 1.0, scale)
    q = np.clip(np.round(w / scale), -127, 127).astype(np.int8)
    return q, scale[..., 0]


def quantize_per_token(x):
    """[GMM] §3.2 activation side: the same symmetric rule applied to every
    row of x [M, K] (one dynamic scale per token)."""
    return quantize_weight_per_channel(x)

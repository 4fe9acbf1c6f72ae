"""Oracle: the grouped GEMMs of the fused MoE (test infrastructure; see
``oracle/__init__.py``).  float64; inputs are taken as the exact values the
GPU receives (bf16 operands are decoded exactly before they get here)."""

import numpy as np


def index_fused_gemm(x, weight, topk_ids):
    """[P1] §03.1-§03.3: out[m, j, :] = x[m] @ weight[topk_ids[m, j]]^T for
    x [M, K], weight [E, N, K] (K contiguous), topk_ids [M, topk]; the result
    is [M, topk, N] with no reduction over j."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ids = np.asarray(topk_ids)
    M, topk = ids.shape
    out = np.zeros((M, topk, w.shape[1]), dtype=np.float64)
    for m in range(M):
        for j in range(topk):
            out[m, j] = x[m] @ w[ids[m, j]].T
    return out


def grouped_gemm_sorted(A, B, sorted_ids, expert_ids, block_m, num_valid,
                        a_row_div, topk_weights=None):
    """[MSG] "fused MoE" (fused_moe_kernel): for every block of block_m
    consecutive entries of sorted_ids, all of expert e = expert_ids[block],
    and every entry p < num_valid in it,
        C[p, :] = A[p // a_row_div, :] @ B[e]^T      (x topk_weights[p] if given).
    Placeholder entries (p >= num_valid) write nothing.  B is [E, N, K].
    Returns C [num_valid, N] in pair order and a bool mask of written rows."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    N = B.shape[1]
    C = np.zeros((num_valid, N), dtype=np.float64)
    written = np.zeros(num_valid, dtype=bool)
    sorted_ids = np.asarray(sorted_ids)
    for blk, e in enumerate(np.asarray(expert_ids)):
        for p in sorted_ids[blk * block_m:(blk + 1) * block_m]:
            p = int(p)
            if p >= num_valid:
                continue
            row = A[p // a_row_div] @ B[int(e)].T
            if topk_weights is not None:
                row = row * float(np.asarray(topk_weights).reshape(-1)[p])
            C[p] = row
            written[p] = True
    return C, written


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)).  The pages use
    silu_and_mul without defining it ([MSG] "参考后端"); this is the plain
    SwiGLU reading."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def silu_and_mul(gate_up):
    """[MSG] "练习" answer 3 and the w1 layout of MoELayer: the first half of
    the last axis is the gate, the second half the up projection; the result
    is silu(gate) * up."""
    gu = np.asarray(gate_up, dtype=np.float64)
    half = gu.shape[-1] // 2
    return silu(gu[..., :half]) * gu[..., half:]

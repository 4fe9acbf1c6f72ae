"""Pins of the alignment, grouped-GEMM, layer and GMM oracles."""

import json
import os

import numpy as np
import pytest

import oracle


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Alignment.

def test_msg_align_printout(golden_dir):
    g = _load(golden_dir, "msg_seeded_example.json")
    s, e, total = oracle.moe_align_block_size(np.array(g["ids"]), g["E"], g["block_m"])
    assert s.tolist() == g["sorted_ids"]
    assert e.tolist() == g["expert_ids"]
    assert total == len(g["sorted_ids"])


def _check_align_invariants(ids, E, B):
    s, eids, total = oracle.moe_align_block_size(ids, E, B)
    flat = np.asarray(ids).reshape(-1)
    P = flat.size
    assert total % B == 0 and s.size == total and eids.size == total // B
    assert total <= oracle.align_max_padded(P, E, B)
    real = s[s < P]
    assert sorted(real.tolist()) == list(range(P))          # each pair once
    for blk in range(total // B):
        seg = s[blk * B:(blk + 1) * B]
        for p in seg[seg < P]:
            assert flat[p] == eids[blk]                      # block's expert
    assert (np.diff(eids) >= 0).all()                        # expert order
    for e in np.unique(eids):
        rows = np.concatenate([s[b * B:(b + 1) * B] for b in np.flatnonzero(eids == e)])
        v = rows[rows < P]
        assert (np.diff(v) > 0).all()                        # stable order
        # valid entries first, then placeholders only
        assert (rows[:v.size] < P).all() and (rows[v.size:] == P).all()
        assert rows.size - v.size < B                        # minimal padding
    return s, eids, total


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("B", [1, 4, 16, 64])
def test_align_invariants_random(seed, B):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 40))
    T = int(rng.integers(1, 50))
    K = int(rng.integers(1, min(E, 4) + 1))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    _check_align_invariants(ids, E, B)


def test_align_matches_rank_count():
    """Cross-formulation written from the definition, pair by pair: pair i of
    expert e lands at (sum over experts e' < e of count(e') rounded up to a
    multiple of B) + (number of pairs j < i with the same expert); every
    other entry is a placeholder, and block b's expert is the expert whose
    padded segment covers position b * B."""
    rng = np.random.default_rng(3)
    for E, B, T, K in [(13, 8, 57, 3), (5, 1, 9, 2), (40, 16, 31, 4), (3, 64, 100, 1)]:
        ids = rng.integers(0, E, size=(T, K))
        flat = [int(v) for v in ids.reshape(-1)]
        P = len(flat)
        count = [flat.count(e) for e in range(E)]
        padded = [-(-c // B) * B for c in count]
        start = [sum(padded[:e]) for e in range(E)]
        total = sum(padded)
        ref = [P] * total
        for i, e in enumerate(flat):
            ref[start[e] + sum(1 for j in range(i) if flat[j] == e)] = i
        ref_e = [next(e for e in range(E) if start[e] <= b * B < start[e] + padded[e])
                 for b in range(total // B)]
        s, eids, got_total = oracle.moe_align_block_size(ids, E, B)
        assert got_total == total and s.tolist() == ref and eids.tolist() == ref_e


def test_align_max_padded_values():
    """Hand-computed values of the padded-length bound P + min(E, P)(B - 1),
    rounded up to a whole block."""
    cases = [  # (pairs, experts, block, bound)
        (0, 8, 4, 0),          # nothing to place
        (5, 8, 4, 20),         # five singleton experts, each padded to 4
        (5, 2, 4, 12),         # 5 + 2 * 3 = 11, rounded up to 12
        (128, 8, 16, 256),     # tiny layer: 128 + 8 * 15 = 248, rounded up to 256
        (32768, 128, 128, 49024),   # prefill: 32768 + 128 * 127 = 49024
        (128, 256, 64, 8192),  # decode T = 16: every pair may sit alone
        (1, 1, 1, 1),
        (7, 3, 1, 7),          # block 1: no padding at all
    ]
    for P, E, B, want in cases:
        assert oracle.align_max_padded(P, E, B) == want, (P, E, B)


def test_align_max_padded_brute_force():
    """Against every assignment of P pairs to E experts on tiny sizes: the
    bound is never exceeded, and it is reached whenever it can be (E >= P,
    or P - E a multiple of B, which lets every used expert hold 1 mod B)."""
    import itertools
    for P in range(0, 6):
        for E in range(1, 5):
            for B in (1, 2, 3, 4):
                best = 0
                for assign in itertools.product(range(E), repeat=P):
                    _, _, total = oracle.moe_align_block_size(
                        np.array(assign, dtype=np.int64).reshape(-1, 1), E, B)
                    best = max(best, total)
                bound = oracle.align_max_padded(P, E, B)
                assert best <= bound
                if E >= P or (P - E) % B == 0:
                    assert best == bound, (P, E, B, best, bound)


def test_align_empty_and_single():
    s, e, total = oracle.moe_align_block_size(np.zeros((0, 2), np.int64), 4, 16)
    assert total == 0 and s.size == 0 and e.size == 0
    s, e, total = oracle.moe_align_block_size(np.array([[3]]), 4, 16)
    assert total == 16 and s[0] == 0 and (s[1:] == 1).all() and e.tolist() == [3]


# ---------------------------------------------------------------------------
# Grouped GEMM: worked example of the index-fused kernel page.

def _p1(golden_dir):
    g = _load(golden_dir, "p1_worked_example.json")
    W = np.zeros((g["E"], g["N"], g["K"]))
    for e, v in enumerate(g["expert_fill"]):
        W[e] = v
    return g, np.array(g["x"], dtype=np.float64), W, np.array(g["topk_ids"])


def test_p1_worked_example(golden_dir):
    g, x, W, ids = _p1(golden_dir)
    out = oracle.index_fused_gemm(x, W, ids)
    assert out.tolist() == g["output"]


@pytest.mark.parametrize("B", [1, 2, 4, 16])
def test_p1_example_through_sorted_gemm(golden_dir, B):
    g, x, W, ids = _p1(golden_dir)
    s, e, total = oracle.moe_align_block_size(ids, g["E"], B)
    C, written = oracle.grouped_gemm_sorted(x, W, s, e, B, ids.size, g["topk"])
    assert written.all()
    assert C.reshape(g["M"], g["topk"], g["N"]).tolist() == g["output"]


def test_single_expert_gemm_is_dense():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((9, 5))
    Bw = rng.standard_normal((1, 6, 5))
    ids = np.zeros((9, 1), np.int64)
    s, e, total = oracle.moe_align_block_size(ids, 1, 4)
    C, _ = oracle.grouped_gemm_sorted(A, Bw, s, e, 4, 9, 1)
    np.testing.assert_allclose(C, A @ Bw[0].T, atol=1e-13)


def test_routed_weight_scales_rows():
    rng = np.random.default_rng(5)
    A = rng.standard_normal((4, 3))
    Bw = rng.standard_normal((2, 5, 3))
    ids = np.array([[0], [1], [1], [0]])
    wts = np.array([0.5, 2.0, -1.0, 3.0])
    s, e, _ = oracle.moe_align_block_size(ids, 2, 2)
    C, _ = oracle.grouped_gemm_sorted(A, Bw, s, e, 2, 4, 1, topk_weights=wts)
    for p in range(4):
        np.testing.assert_allclose(C[p], wts[p] * (A[p] @ Bw[ids[p, 0]].T), atol=1e-13)


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.silu(1.0), 1.0 / (1.0 + np.exp(-1.0)), atol=0)
    np.testing.assert_allclose(oracle.silu(50.0), 50.0, rtol=1e-15)
    assert abs(oracle.silu(-50.0)) < 1e-19
    # gate is the FIRST half: silu(1)*2 = 1.4621..., not silu(2)*1 = 1.7616...
    np.testing.assert_allclose(oracle.silu_and_mul(np.array([1.0, 2.0])),
                               2.0 * 0.7310585786300049, rtol=1e-15)


# ---------------------------------------------------------------------------
# Layer.

def _rand_layer(seed, T=11, H=8, I=6, E=5, K=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    w1 = rng.standard_normal((E, 2 * I, H)) * 0.3
    w2 = rng.standard_normal((E, H, I)) * 0.3
    gating = rng.standard_normal((T, E))
    return x, w1, w2, gating


def test_expert_loop_equals_token_loop():
    x, w1, w2, g = _rand_layer(1)
    w, ids = oracle.grouped_topk(g, 2, True, 1, 1)
    a = oracle.moe_layer_expert_loop(x, w1, w2, w, ids)
    b = oracle.moe_layer_token_loop(x, w1, w2, w, ids)
    np.testing.assert_allclose(a, b, atol=1e-12, rtol=0)


def test_pair_rows_are_single_slot_layers():
    """Slot k of the pair rows is the token loop run with that slot alone;
    the expert loop is their sum over slots."""
    x, w1, w2, g = _rand_layer(5, K=3)
    w, ids = oracle.grouped_topk(g, 3, True, 1, 1)
    rows = oracle.moe_layer_pair_rows(x, w1, w2, w, ids)
    assert rows.shape == (x.shape[0], 3, x.shape[1])
    for k in range(3):
        one = oracle.moe_layer_token_loop(x, w1, w2, w[:, k:k + 1], ids[:, k:k + 1])
        np.testing.assert_allclose(rows[:, k], one, atol=1e-12, rtol=0)
    np.testing.assert_allclose(rows.sum(axis=1), oracle.moe_layer_expert_loop(x, w1, w2, w, ids),
                               atol=0, rtol=0)


def test_identical_experts_reduce_to_dense():
    """If every expert holds the same weights the renormalised layer is the
    dense SwiGLU MLP, whatever the routing; with a scale it is scaled."""
    x, w1, w2, g = _rand_layer(2)
    w1[:] = w1[0]
    w2[:] = w2[0]
    dense = oracle.dense_swiglu(x, w1[0], w2[0])
    out, w, ids = oracle.moe_forward(x, g, w1, w2, 3, True, 1, 1,
                                     routed_scaling_factor=2.5)
    np.testing.assert_allclose(out, 2.5 * dense, atol=1e-12)


def test_dense_swiglu_against_matmul_chain():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 3))
    w1 = rng.standard_normal((4, 3))     # I = 2
    w2 = rng.standard_normal((3, 2))
    gu = x @ w1.T
    h = gu[:, :2] / (1 + np.exp(-gu[:, :2])) * gu[:, 2:]
    np.testing.assert_allclose(oracle.dense_swiglu(x, w1, w2), h @ w2.T, atol=1e-14)


def test_expert_relabelling_invariance():
    x, w1, w2, g = _rand_layer(3)
    perm = np.random.default_rng(0).permutation(5)
    out, _, _ = oracle.moe_forward(x, g, w1, w2, 2)
    out_p, _, _ = oracle.moe_forward(x, g[:, perm], w1[perm], w2[perm], 2)
    np.testing.assert_allclose(out_p, out, atol=1e-12)


def test_layer_linear_in_routing_weights():
    x, w1, w2, g = _rand_layer(4)
    w, ids = oracle.grouped_topk(g, 2, False, 1, 1)
    a = oracle.moe_layer_expert_loop(x, w1, w2, w, ids)
    b = oracle.moe_layer_expert_loop(x, w1, w2, 3.0 * w, ids)
    np.testing.assert_allclose(b, 3.0 * a, atol=1e-12)


# ---------------------------------------------------------------------------
# GMM and the INT8 variant.

def test_quantizer_closed_form():
    w = np.array([[127.0, 2.5, -2.5, 0.5, 1.5, -127.0]])   # amax 127 -> scale 1
    q, s = oracle.quantize_weight_per_channel(w)
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, 2, -2, 0, 2, -127]]        # half to even
    w = np.array([[0.5, -1.0, 0.25]])
    q, s = oracle.quantize_weight_per_channel(w)
    np.testing.assert_allclose(s, [1.0 / 127.0])
    assert q.tolist() == [[64, -127, 32]]


def test_per_token_quantizer_closed_form():
    """[GMM] §3.2 activation side: one scale per row, amax maps to +-127,
    halves round to even, an all-zero row gets scale 1 and codes 0, and the
    reconstruction error of every element is at most half a step."""
    x = np.array([[254.0, 5.0, -3.0, 1.0],        # scale 2: 127, 2.5->2, -1.5->-2, 0.5->0
                  [0.0, 0.0, 0.0, 0.0],
                  [-0.5, 0.25, 0.125, 0.0]])      # scale 0.5/127
    q, s = oracle.quantize_per_token(x)
    assert s.tolist()[:2] == [2.0, 1.0]
    np.testing.assert_allclose(s[2], 0.5 / 127.0)
    assert q.tolist() == [[127, 2, -2, 0], [0, 0, 0, 0], [-127, 64, 32, 0]]
    rng = np.random.default_rng(9)
    x = rng.standard_normal((16, 40))
    q, s = oracle.quantize_per_token(x)
    assert q.dtype == np.int8 and s.shape == (16,)
    assert (np.abs(q).max(axis=1) == 127).all()
    assert (np.abs(q.astype(np.float64) * s[:, None] - x) <= 0.5 * s[:, None] + 1e-15).all()


def test_gmm_int8_exactly_representable():
    """Weights and activations that are exactly q * scale: the int8 GMM
    equals the float GMM of the dequantised tensors."""
    rng = np.random.default_rng(5)
    E, N, K = 4, 7, 33
    sizes = np.array([0, 5, 1, 9])
    off = np.concatenate([[0], np.cumsum(sizes)])
    M = int(off[-1])
    Xq = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    Wq = rng.integers(-127, 128, size=(E, N, K)).astype(np.int8)
    sx = 2.0 ** rng.integers(-8, 0, size=M)
    sw = 2.0 ** rng.integers(-10, -2, size=(E, N))
    Y = oracle.gmm_int8(Xq, Wq, sx, sw, off)
    X = Xq * sx[:, None]
    W = Wq * sw[:, :, None]
    np.testing.assert_allclose(Y, oracle.gmm(X, W, off), rtol=1e-15, atol=0)
    # rows of each group used that group's weights
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            np.testing.assert_allclose(Y[lo:hi], X[lo:hi] @ W[e].T, rtol=1e-15)


def test_gmm_int8_extreme_accumulation():
    K = 4096
    Xq = np.full((2, K), 127, np.int8)
    Xq[1] = -127
    Wq = np.full((1, 3, K), -127, np.int8)
    Y = oracle.gmm_int8(Xq, Wq, np.ones(2), np.ones((1, 3)), np.array([0, 2]))
    assert Y[0].tolist() == [-66064384.0] * 3
    assert Y[1].tolist() == [66064384.0] * 3


def test_gmm_int8_sum_equals_int64_sum():
    """The float64 integer sums equal exact int64 sums (random int8 data)."""
    rng = np.random.default_rng(6)
    Xq = rng.integers(-127, 128, size=(7, 512)).astype(np.int8)
    Wq = rng.integers(-127, 128, size=(2, 9, 512)).astype(np.int8)
    off = np.array([0, 3, 7])
    Y = oracle.gmm_int8(Xq, Wq, np.ones(7), np.ones((2, 9)), off)
    for e in range(2):
        exact = Xq[off[e]:off[e + 1]].astype(np.int64) @ Wq[e].astype(np.int64).T
        assert (Y[off[e]:off[e + 1]] == exact).all()

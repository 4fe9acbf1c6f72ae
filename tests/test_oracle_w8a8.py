"""Pins of the oracle's INT8-weight, INT8-activation fused-MoE layer and of
its float32 row quantiser (no GPU)."""

import numpy as np

import oracle


def test_quantize_rows_f32_closed_form():
    """[GMM] §3.2: scale = amax / 127 and round half to even, in float32."""
    x = np.array([[254.0, 5.0, -3.0, 1.0, -254.0],     # scale 2: 2.5 -> 2, -1.5 -> -2, 0.5 -> 0
                  [0.0, 0.0, 0.0, 0.0, 0.0],           # all zero: scale 1, codes 0
                  [127.0, 63.5, -0.5, 0.25, 1.5]],     # scale 1: 63.5 -> 64, -0.5 -> -0, 1.5 -> 2
                 dtype=np.float32)
    q, s = oracle.quantize_rows_f32(x)
    assert s.dtype == np.float32 and q.dtype == np.int8
    assert s.tolist() == [2.0, 1.0, 1.0]
    assert q.tolist() == [[127, 2, -2, 0, -127], [0, 0, 0, 0, 0], [127, 64, 0, 0, 2]]


def test_quantize_rows_f32_bounds():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((50, 77)) * rng.uniform(1e-3, 1e3, size=(50, 1))).astype(np.float32)
    q, s = oracle.quantize_rows_f32(x)
    assert (np.abs(q).max(axis=1) == 127).all()
    err = np.abs(q.astype(np.float64) * s[:, None].astype(np.float64) - x.astype(np.float64))
    assert (err <= 0.5 * s[:, None] * (1 + 1e-6)).all()


def _case(seed, T=23, H=48, I=40, E=5, K=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    w1 = rng.standard_normal((E, 2 * I, H)) * 0.1
    w2 = rng.standard_normal((E, H, I)) * 0.1
    w1q, s1 = oracle.quantize_weight_per_channel(w1)
    w2q, s2 = oracle.quantize_weight_per_channel(w2)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    wts = rng.random((T, K))
    return x, w1q, s1, w2q, s2, wts, ids


def test_w8a8_expert_loop_equals_token_loop():
    x, w1q, s1, w2q, s2, wts, ids = _case(1)
    a = oracle.moe_layer_w8a8_expert_loop(x, w1q, s1, w2q, s2, wts, ids)
    b = oracle.moe_layer_w8a8_token_loop(x, w1q, s1, w2q, s2, wts, ids)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(a).max())


def test_w8a8_single_expert_is_two_int8_gmms():
    """E = 1: the layer is gmm_int8 -> silu*up -> per-row quantise ->
    gmm_int8, times the routing weight (composed from separately pinned
    oracle functions)."""
    x, w1q, s1, w2q, s2, wts, _ = _case(3, E=1, K=1)
    T = x.shape[0]
    ids = np.zeros((T, 1), np.int64)
    out = oracle.moe_layer_w8a8_expert_loop(x, w1q, s1, w2q, s2, wts, ids)
    xq, sx = oracle.quantize_rows_f32(x)
    off = np.array([0, T])
    h = oracle.silu_and_mul(oracle.gmm_int8(xq, w1q, sx, s1, off))
    hq, sh = oracle.quantize_rows_f32(h)
    ref = oracle.gmm_int8(hq, w2q, sh, s2, off) * wts
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=0)


def test_w8a8_close_to_float_layer():
    """Quantisation error only: against the float layer on the dequantised
    weights and the unquantised activations."""
    x, w1q, s1, w2q, s2, wts, ids = _case(5, T=64, H=128, I=96, E=6, K=3)
    q = oracle.moe_layer_w8a8_expert_loop(x, w1q, s1, w2q, s2, wts, ids)
    w1 = w1q * s1[..., None]
    w2 = w2q * s2[..., None]
    f = oracle.moe_layer_expert_loop(x.astype(np.float64), w1, w2, wts, ids)
    err = np.abs(q - f).max() / np.abs(f).max()
    assert err < 2e-2, err
    # dropping any one scale would change the result by orders of magnitude
    assert np.abs(q).max() / np.abs(f).max() < 1.05


def test_w8a8_linear_in_routing_weights():
    x, w1q, s1, w2q, s2, wts, ids = _case(7)
    a = oracle.moe_layer_w8a8_expert_loop(x, w1q, s1, w2q, s2, wts, ids)
    b = oracle.moe_layer_w8a8_expert_loop(x, w1q, s1, w2q, s2, 2.5 * wts, ids)
    np.testing.assert_allclose(b, 2.5 * a, rtol=1e-12)

"""GPU parity of the int8 path: moe_quantize_rows bit for bit against the
oracle's float32 quantiser, and moe_forward_w8a8 (int8 weights and
activations in both GEMMs) against the oracle's int8 layer.  Bar for the
layer: max-abs-rel 3e-2 (the int8 bar)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bf16_dev, layer_inputs, require_gpu
from parity import BAR_INT8, check_routing, max_abs_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols,ld", [
    (37, 64, 64), (5, 2048, 2048), (9, 200, 264),   # 32 lanes per row / 64 lanes
    (11, 768, 768), (6, 1024, 1040), (7, 1536, 1536),   # 3 chunks per lane; 64 lanes x 2, x 3
    (3, 2056, 2056)])                                  # past 2048 columns: read twice
def test_quantize_rows_bit_exact(moe, dev, dtype, rows, cols, ld):
    rng = np.random.default_rng(rows * cols + ld)
    x = (rng.standard_normal((rows, ld)) * rng.uniform(1e-3, 1e3, (rows, 1))).astype(np.float32)
    x[1] = 0.0                                    # all-zero row
    x[2, :4] = [254.0, 5.0, -3.0, 1.0]            # halfway codes (scale 2)
    x[2, 4:] = 0.0
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(x)
        xd = bf16_dev(bits, dev)
        xh = oracle.bf16_bits_to_f64(bits).astype(np.float32)   # exact
    else:
        xd = torch.from_numpy(x).to(dev)
        xh = x
    q, s = moe.moe_quantize_rows(xd[:, :cols] if ld == cols else _strided(xd, cols))
    torch.cuda.synchronize()
    qr, sr = oracle.quantize_rows_f32(xh[:, :cols])
    assert (s.cpu().numpy() == sr).all()
    assert (q.cpu().numpy() == qr).all()


def _strided(xd, cols):
    """A [rows, cols] view with row stride ld (the binding passes stride(0))."""
    return xd.as_strided((xd.shape[0], cols), (xd.shape[1], 1))


def _quantized_weights(d):
    """Per-channel int8 weights of the layer (input preparation, on the host
    from the exact bf16 values)."""
    w1q, s1 = oracle.quantize_weight_per_channel(d["w1_host"])
    w2q, s2 = oracle.quantize_weight_per_channel(d["w2_host"])
    return w1q, s1, w2q, s2


def _dev(moe, dev, w1q, s1, w2q, s2, layout):
    w1 = torch.from_numpy(w1q).to(dev)
    w2 = torch.from_numpy(w2q).to(dev)
    if layout == "packed":
        w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
    return (w1, torch.from_numpy(s1.astype(np.float32)).to(dev), w2,
            torch.from_numpy(s2.astype(np.float32)).to(dev))


@pytest.mark.parametrize("layout,block_m", [("plain", 0), ("packed", 0), ("packed", 64),
                                            ("plain", 128), ("packed", 256)])
def test_w8a8_tiny_layer(moe, dev, layout, block_m):
    cfg = synth.CONFIGS["tiny"]
    d = layer_inputs(cfg, dev, x_dtype="bf16")
    w1q, s1, w2q, s2 = _quantized_weights(d)
    W1, S1, W2, S2 = _dev(moe, dev, w1q, s1, w2q, s2, layout)
    ids = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device=dev)
    w = torch.empty((cfg.T, cfg.topk), dtype=torch.float32, device=dev)
    out = moe.moe_forward_w8a8(d["x"], d["gating"], W1, S1, W2, S2, cfg.topk, block_m=block_m,
                               topk_weights_out=w, topk_ids_out=ids)
    torch.cuda.synchronize()
    w_ref, ids_ref = oracle.grouped_topk(d["gating_host"], cfg.topk)
    assert (ids.cpu().numpy() == ids_ref).all()
    ref = oracle.moe_layer_w8a8_expert_loop(d["x_host"], w1q, s1, w2q, s2, w_ref, ids_ref)
    got = out.float().cpu().numpy()
    err = max_abs_rel(got, ref)
    print("w8a8 tiny layer (%s, block_m %d) err=%.3e" % (layout, block_m, err))
    assert np.isfinite(got).all() and err <= BAR_INT8


class _Int8Experts:
    """One expert's int8 weights (and f32 scales) pulled from the device on
    demand, for the oracle at full layer sizes."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return self.t[int(e)].cpu().numpy()


def _device_quantize(w):
    """Per-output-channel int8 of a device bf16 [E, N, K] tensor, one expert
    at a time (input preparation; same rule as the oracle's quantiser)."""
    E, N, K = w.shape
    q = torch.empty((E, N, K), dtype=torch.int8, device=w.device)
    s = torch.empty((E, N), dtype=torch.float32, device=w.device)
    for e in range(E):
        we = w[e].double()
        amax = we.abs().amax(dim=1, keepdim=True)
        se = torch.where(amax == 0, torch.ones_like(amax), amax / 127.0)
        q[e] = torch.clamp(torch.round(we / se), -127, 127).to(torch.int8)
        s[e] = se.squeeze(1).float()
    return q, s


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["prefill", "decode16", "decode64"])
def test_w8a8_layer_full(moe, dev, name):
    """Every output row of the int8 layer at the prefill and decode (T=16 and
    T=64) shapes, packed weights, against the oracle's int8 layer run on the
    routing the GPU accepted (itself checked against the oracle's)."""
    cfg = synth.CONFIGS[name]
    d = layer_inputs(cfg, dev)
    w1q, s1 = _device_quantize(d["w1"])
    w2q, s2 = _device_quantize(d["w2"])
    del d["w1"], d["w2"]
    torch.cuda.empty_cache()
    p1, p2 = moe.moe_pack_weights(w1q, "silu_mul"), moe.moe_pack_weights(w2q, "none")
    T, K = cfg.T, cfg.topk
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    out = moe.moe_forward_w8a8(d["x"], d["gating"], p1, s1, p2, s2, K, cfg.groups,
                               cfg.topk_group, "softmax", cfg.renormalize, cfg.scale,
                               topk_weights_out=w, topk_ids_out=ids)
    torch.cuda.synchronize()
    wn, idn = w.cpu().numpy(), ids.cpu().numpy()
    check_routing(wn, idn, d["gating_host"], K, cfg.renormalize, cfg.groups, cfg.topk_group,
                  "softmax", cfg.scale)
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    ref = oracle.moe_layer_w8a8_expert_loop(
        d["x_host"], _Int8Experts(w1q), _Int8Experts(s1), _Int8Experts(w2q),
        _Int8Experts(s2), wn.astype(np.float64), idn)
    err = max_abs_rel(o, ref)
    print("w8a8 %s, all rows: err=%.3e" % (name, err))
    assert err <= BAR_INT8


@pytest.mark.parametrize("case", ["prefill", "ragged", "big_expert"])
def test_w8a8_wide_tiles_match_tile_kernels(moe, dev, case):
    """moe_forward_w8a8 on the expert-wide int8 tiles (block_m 32) gives the
    same bits as on the 256 x 128 tiles (block_m 128): the int32 sums are
    exact and the epilogues apply the same scales in the same order.  At the
    prefill size (the automatic choice), with H and I not multiples of the
    tiles, and with one expert of 700 pairs split over three tiles; both
    weight layouts."""
    from synth.configs import Config
    if case == "prefill":
        cfg = synth.CONFIGS["prefill"]
        assert moe.moe_forward_block_m(cfg.T, cfg.E, cfg.topk, "bf16", "packed") == 32
    elif case == "ragged":
        cfg = Config(31, "w8a8 ragged", T=333, H=272, I=160, E=40, topk=6, groups=8,
                     topk_group=3, x_dtype="bf16", w_std=0.05)
    else:
        cfg = Config(32, "w8a8 big expert", T=700, H=256, I=384, E=8, topk=1, x_dtype="bf16",
                     w_std=0.05)
    d = layer_inputs(cfg, dev)
    g = d["gating"]
    if case == "big_expert":
        g = g.clone()
        g[:, 5] += 8.0
    w1q, s1 = _device_quantize(d["w1"])
    w2q, s2 = _device_quantize(d["w2"])
    layouts = ["packed"] if case == "prefill" else ["plain", "packed"]
    for layout in layouts:
        q1, q2 = w1q, w2q
        if layout == "packed":
            q1, q2 = moe.moe_pack_weights(w1q, "silu_mul"), moe.moe_pack_weights(w2q, "none")
        outs = []
        for bm in (32, 128):
            outs.append(moe.moe_forward_w8a8(d["x"], g, q1, s1, q2, s2, cfg.topk, cfg.groups,
                                             cfg.topk_group, "softmax", cfg.renormalize,
                                             cfg.scale, block_m=bm))
        torch.cuda.synchronize()
        nd = int((outs[0].view(torch.int16) != outs[1].view(torch.int16)).sum())
        print("w8a8 %s %s: %d of %d outputs differ" % (case, layout, nd, outs[0].numel()))
        assert nd == 0

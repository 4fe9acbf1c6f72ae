"""GPU parity of the whole layer, moe_forward, against the oracle, every
output row: the tiny layer, the prefill layer (T=4096, H=2048, I=768, E=128,
top-8) and the decode layers (T=16 and 64, H=7168, I=2048, E=256, grouped
top-8) at full size, in the launch configuration the benchmark times and in
the other kernel variants.  Bar: max-abs-rel 2e-2."""

import time

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import layer_inputs, require_gpu, bf16_host_f64
from parity import BAR_BF16, check_routing, max_abs_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


def _packed(moe, d):
    """The layer's weights in the packed layout (cached in the input dict)."""
    if "w1_packed" not in d:
        d["w1_packed"] = moe.moe_pack_weights(d["w1"], "silu_mul")
        d["w2_packed"] = moe.moe_pack_weights(d["w2"], "none")
    return d["w1_packed"], d["w2_packed"]


def _run(moe, cfg, d, block_m=0, dev=None, layout="plain"):
    T, E, K = cfg.T, cfg.E, cfg.topk
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w1, w2 = _packed(moe, d) if layout == "packed" else (d["w1"], d["w2"])
    out = moe.moe_forward(d["x"], d["gating"], w1, w2, K, cfg.groups,
                          cfg.topk_group, "softmax", cfg.renormalize, cfg.scale,
                          block_m=block_m, topk_weights_out=w, topk_ids_out=ids)
    torch.cuda.synchronize()
    return out, w.cpu().numpy(), ids.cpu().numpy()


def _out_host(out):
    return out.cpu().numpy().astype(np.float64) if out.dtype == torch.float32 \
        else bf16_host_f64(out)


def _oracle_rows(cfg, d, rows, w_gpu=None, ids_gpu=None):
    """Oracle output for the given token rows (routing recomputed per row;
    where a near-tie was accepted, the oracle re-runs with the GPU's ids)."""
    g = d["gating_host"][rows]
    w, ids = oracle.grouped_topk(g, cfg.topk, cfg.renormalize, cfg.groups, cfg.topk_group,
                                 "softmax", cfg.scale)
    if ids_gpu is not None:
        for i, r in enumerate(rows):
            if not (ids_gpu[r] == ids[i]).all():
                ids[i] = ids_gpu[r]
                s = oracle.softmax_scores(g[i:i + 1])[0, ids[i]]
                w[i] = (s / s.sum() if cfg.renormalize else s) * cfg.scale
    return oracle.moe_layer_expert_loop(d["x_host"][rows], d["w1_host"], d["w2_host"], w, ids)


@pytest.mark.parametrize("block_m", [0, 16, 32, 64, 128])
def test_tiny_layer(moe, dev, block_m):
    cfg = synth.CONFIGS["tiny"]
    d = layer_inputs(cfg, dev)
    out, w, ids = _run(moe, cfg, d, block_m, dev)
    assert out.dtype == torch.float32 and out.shape == (cfg.T, cfg.H)
    check_routing(w, ids, d["gating_host"], cfg.topk, True, 1, 1, "softmax", 1.0)
    ref = oracle.moe_layer_expert_loop(d["x_host"], d["w1_host"], d["w2_host"],
                                       *oracle.grouped_topk(d["gating_host"], cfg.topk))
    err = max_abs_rel(out.cpu().numpy(), ref)
    print("tiny layer block_m=%d err=%.3e" % (block_m, err))
    assert err <= BAR_BF16


@pytest.mark.parametrize("block_m,layout", [(16, "plain"), (32, "plain"), (128, "plain"),
                                            (256, "plain"), (0, "packed"), (32, "packed"),
                                            (64, "packed"), (128, "packed"), (256, "packed")])
def test_tiny_layer_bf16_x(moe, dev, block_m, layout):
    cfg = synth.CONFIGS["tiny"]
    d = layer_inputs(cfg, dev, x_dtype="bf16")
    out, w, ids = _run(moe, cfg, d, block_m, dev, layout)
    assert out.dtype == torch.bfloat16
    ref = oracle.moe_layer_expert_loop(d["x_host"], d["w1_host"], d["w2_host"],
                                       *oracle.grouped_topk(d["gating_host"], cfg.topk))
    assert max_abs_rel(_out_host(out), ref) <= BAR_BF16


def test_single_expert_is_dense(moe, dev):
    """E = 1, top-1: the layer is the dense SwiGLU MLP."""
    from synth.configs import Config
    cfg = Config(11, "dense", T=37, H=64, I=96, E=1, topk=1, x_dtype="bf16", w_std=0.1)
    d = layer_inputs(cfg, dev)
    for bm in (16, 64, 256):
        out, w, ids = _run(moe, cfg, d, bm, dev)
        assert (ids == 0).all() and np.allclose(w, 1.0)
        ref = oracle.dense_swiglu(d["x_host"], d["w1_host"][0], d["w2_host"][0])
        assert max_abs_rel(_out_host(out), ref) <= BAR_BF16


@pytest.fixture(scope="module")
def prefill_inputs(dev):
    return layer_inputs(synth.CONFIGS["prefill"], dev)


# Oracle outputs of whole layers, keyed by config; recomputed only if a later
# run accepted different near-tie ids.
_ORACLE_ALL = {}


def _oracle_all(cfg, d, w, ids):
    hit = _ORACLE_ALL.get(cfg.name)
    if hit is None or not (hit[0] == ids).all():
        t0 = time.time()
        ref = _oracle_rows(cfg, d, np.arange(cfg.T), w, ids)
        print("oracle %s, all %d rows: %.1f s" % (cfg.name, cfg.T, time.time() - t0), flush=True)
        _ORACLE_ALL[cfg.name] = hit = (ids.copy(), ref)
    return hit[1]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layout", ["packed", "plain"])
def test_prefill_layer_full(moe, dev, prefill_inputs, layout):
    """Every one of the 4096 output rows against the oracle, in the
    benchmark's configuration (packed weights, automatic block size) and on
    plain weights."""
    cfg = synth.CONFIGS["prefill"]
    d = prefill_inputs
    out, w, ids = _run(moe, cfg, d, 0, dev, layout)
    check_routing(w, ids, d["gating_host"], cfg.topk, True, 1, 1, "softmax", 1.0)
    o = _out_host(out)
    assert np.isfinite(o).all()
    err = max_abs_rel(o, _oracle_all(cfg, d, w, ids))
    print("prefill %s, all rows: err=%.3e" % (layout, err))
    assert err <= BAR_BF16


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode16", "decode64"])
def test_decode_layer_full(moe, dev, name):
    """Every output row of the decode layers against the oracle (touched
    experts decoded one at a time): the tile kernels on plain weights (the
    automatic block size), the weight-streaming kernel (block_m 16) and the
    tile kernels on packed weights (the benchmark's configuration)."""
    cfg = synth.CONFIGS[name]
    d = layer_inputs(cfg, dev)
    out, w, ids = _run(moe, cfg, d, 0, dev)
    check_routing(w, ids, d["gating_host"], cfg.topk, True, cfg.groups, cfg.topk_group,
                  "softmax", cfg.scale)
    np.testing.assert_allclose(w.sum(1), cfg.scale, rtol=1e-5)
    assert moe.moe_forward_block_m(cfg.T, cfg.E, cfg.topk) == 64   # the tile kernels
    ref = _oracle_all(cfg, d, w, ids)
    outs = {"tile, plain": out}
    outs["stream, block_m 16"], _, ids_s = _run(moe, cfg, d, 16, dev)
    outs["tile, packed"], _, ids_p = _run(moe, cfg, d, 0, dev, "packed")
    assert (ids_s == ids).all() and (ids_p == ids).all()
    del d["w1_packed"], d["w2_packed"]
    for k, o in outs.items():
        oh = _out_host(o)
        assert np.isfinite(oh).all()
        err = max_abs_rel(oh, ref)
        print("%s %s, all rows: err=%.3e" % (name, k, err))
        assert err <= BAR_BF16, k


@pytest.mark.parametrize("block_m", [32, 64, 128, 256])
def test_layer_reuses_workspace(moe, dev, block_m):
    """Consecutive layers on one workspace that starts full of garbage, with
    different tokens and sizes: no call reads another call's alignment, h or
    y."""
    from synth.configs import Config
    cfgs = [Config(12, "reuse", T=T, H=256, I=384, E=16, topk=4, x_dtype="bf16", w_std=0.05,
                   extra={"sub": i}) for i, T in enumerate([600, 150, 601])]
    need = max(moe.moe_forward_workspace_size(c.T, c.H, c.I, c.E, c.topk, block_m) for c in cfgs)
    ws = torch.full((need,), 0x5a, dtype=torch.uint8, device=dev)
    for c in cfgs:
        d = layer_inputs(c, dev)
        ref = oracle.moe_layer_expert_loop(d["x_host"], d["w1_host"], d["w2_host"],
                                           *oracle.grouped_topk(d["gating_host"], c.topk))
        for layout in ("plain", "packed"):
            w1, w2 = _packed(moe, d) if layout == "packed" else (d["w1"], d["w2"])
            out = moe.moe_forward(d["x"], d["gating"], w1, w2, c.topk, block_m=block_m,
                                  workspace=ws)
            torch.cuda.synchronize()
            err = max_abs_rel(_out_host(out), ref)
            print("reuse T=%d %s block_m %d err=%.3e" % (c.T, layout, block_m, err))
            assert err <= BAR_BF16


# ---- small layers: routing, then one launch for the GEMMs and the sum ----

def _small_case(cfg, dev, x_dtype=None, bias_expert=None):
    d = layer_inputs(cfg, dev, x_dtype=x_dtype)
    if bias_expert is not None:   # every token's best expert is the same one
        g = d["gating_host"].astype(np.float32)
        g[:, bias_expert] += np.float32(8.0)
        d["gating_host"] = g.astype(np.float64)
        d["gating"] = torch.from_numpy(g).to(dev)
    return d


def _check_small(moe, cfg, d, dev):
    out, w, ids = _run(moe, cfg, d, 0, dev)
    check_routing(w, ids, d["gating_host"], cfg.topk, cfg.renormalize, cfg.groups,
                  cfg.topk_group, "softmax", cfg.scale)
    ref = _oracle_rows(cfg, d, np.arange(cfg.T), w, ids)
    err = max_abs_rel(_out_host(out), ref)
    print("small layer %s err=%.3e" % (cfg.name, err))
    assert err <= BAR_BF16
    return out


@pytest.mark.parametrize("case", ["tiny_bf16", "skewed", "dense", "grouped", "max_pairs",
                                  "past_limit"])
def test_small_layer_shapes(moe, dev, case):
    """Automatic block size with plain weights: layers up to 2048 pairs (and
    6 * pairs * H * I up to 2^28) run as routing plus one launch, one
    workgroup per token; larger ones take the aligned path.  Covers one
    expert with all the tokens, empty experts, E = 1 with H / 8 and I / 8 not
    powers of two, grouped routing with a scale, the pair limit and just
    past it."""
    from synth.configs import Config
    x_dtype = None
    bias = None
    if case == "tiny_bf16":
        cfg, x_dtype = synth.CONFIGS["tiny"], "bf16"
    elif case == "skewed":
        cfg, bias = Config(13, "skewed", T=64, H=128, I=256, E=8, topk=2, x_dtype="f32"), 3
    elif case == "dense":
        cfg = Config(14, "dense", T=37, H=64, I=96, E=1, topk=1, x_dtype="f32", w_std=0.1)
    elif case == "grouped":
        cfg = Config(15, "grouped", T=50, H=64, I=128, E=64, topk=6, groups=8, topk_group=2,
                     scale=2.5, x_dtype="bf16", w_std=0.05)
    elif case == "max_pairs":
        cfg = Config(16, "max pairs", T=256, H=128, I=128, E=32, topk=8, x_dtype="f32")
    else:
        cfg = Config(17, "past the pair limit", T=257, H=128, I=128, E=32, topk=8, x_dtype="f32")
    d = _small_case(cfg, dev, x_dtype, bias)
    _check_small(moe, cfg, d, dev)


def test_small_layer_repeatable_on_garbage_workspace(moe, dev):
    """A workspace full of garbage works, and repeated calls give identical
    bits (fixed summation order)."""
    cfg = synth.CONFIGS["tiny"]
    d = layer_inputs(cfg, dev)
    ws = torch.full((moe.moe_forward_workspace_size(cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk),),
                    0x7f, dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(3):
        outs.append(moe.moe_forward(d["x"], d["gating"], d["w1"], d["w2"], cfg.topk,
                                    workspace=ws).cpu())
        torch.cuda.synchronize()
    ref = oracle.moe_layer_expert_loop(d["x_host"], d["w1_host"], d["w2_host"],
                                       *oracle.grouped_topk(d["gating_host"], cfg.topk))
    assert max_abs_rel(outs[0].numpy(), ref) <= BAR_BF16
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("scoring,renorm,scale", [("sigmoid", True, 1.0), ("sigmoid", False, 2.5),
                                                  ("softmax", False, 1.5)])
@pytest.mark.parametrize("block_m", [0, 32, 128])
def test_layer_routing_variants(moe, dev, scoring, renorm, scale, block_m):
    """The whole layer with the other routing variants (sigmoid scores, no
    renormalisation, a scale): moe_forward's own routing is checked against
    the oracle's (near-tie rule), and its output against the oracle layer run
    with the routing it accepted, in full, on both weight layouts."""
    from synth.configs import Config
    cfg = Config(14, "variants", T=300, H=256, I=384, E=64, topk=6, groups=8, topk_group=3,
                 x_dtype="bf16", w_std=0.05, scale=scale, renormalize=renorm,
                 extra={"sub": ["sigmoid", "softmax"].index(scoring) * 2 + int(renorm)})
    d = layer_inputs(cfg, dev)
    for layout in ("plain", "packed"):
        w1, w2 = _packed(moe, d) if layout == "packed" else (d["w1"], d["w2"])
        w = torch.empty((cfg.T, cfg.topk), dtype=torch.float32, device=dev)
        ids = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device=dev)
        out = moe.moe_forward(d["x"], d["gating"], w1, w2, cfg.topk, cfg.groups, cfg.topk_group,
                              scoring, renorm, scale, block_m=block_m, topk_weights_out=w,
                              topk_ids_out=ids)
        torch.cuda.synchronize()
        wn, idn = w.cpu().numpy(), ids.cpu().numpy()
        check_routing(wn, idn, d["gating_host"], cfg.topk, renorm, cfg.groups, cfg.topk_group,
                      scoring, scale)
        ref = oracle.moe_layer_expert_loop(d["x_host"], d["w1_host"], d["w2_host"],
                                           wn.astype(np.float64), idn)
        err = max_abs_rel(_out_host(out), ref)
        print("%s renorm=%s scale=%.1f block_m %d %s err=%.3e" % (scoring, renorm, scale, block_m,
                                                                 layout, err))
        assert err <= BAR_BF16


def test_layers_with_zero_tokens(moe, dev):
    """T = 0: both layer calls return an empty output without launching,
    for bf16 and f32 tokens and both weight layouts."""
    E, H, I, K = 16, 256, 384, 4
    g = torch.empty((0, E), dtype=torch.float32, device=dev)
    w1 = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((E, H, I), dtype=torch.bfloat16, device=dev)
    packed = (moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none"))
    for dtype in (torch.bfloat16, torch.float32):
        x = torch.empty((0, H), dtype=dtype, device=dev)
        for ws in ((w1, w2), packed) if dtype == torch.bfloat16 else ((w1, w2),):
            out = moe.moe_forward(x, g, ws[0], ws[1], K)
            assert out.shape == (0, H) and out.dtype == dtype
    q1 = torch.zeros((E, 2 * I, H), dtype=torch.int8, device=dev)
    q2 = torch.zeros((E, H, I), dtype=torch.int8, device=dev)
    s1 = torch.ones((E, 2 * I), dtype=torch.float32, device=dev)
    s2 = torch.ones((E, H), dtype=torch.float32, device=dev)
    out = moe.moe_forward_w8a8(torch.empty((0, H), dtype=torch.bfloat16, device=dev), g, q1, s1,
                               q2, s2, K)
    torch.cuda.synchronize()
    assert out.shape == (0, H)

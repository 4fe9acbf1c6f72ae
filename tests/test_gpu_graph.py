"""The layer calls inside a HIP graph.  moe_forward (the tiny layer's
one-launch path, the decode tile kernels and the prefill expert-wide
kernels), moe_forward_noalloc and moe_forward_w8a8 are captured once with
torch.cuda.graph and replayed several times, with other eager layer calls
and synchronisations between the replays.  Every replay must give the bits
of the eager call on the same inputs, also after the inputs were overwritten
in place between replays (the graph reads the live buffers).  The library
enqueues kernels only (no memset or copy nodes), and every kernel is
deterministic, so the comparison is bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bf16_dev, layer_inputs, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


def _second_inputs(cfg, d, dev):
    """Another x and gating of the same shapes and dtypes (seeded apart)."""
    T, H, E = cfg.T, cfg.H, cfg.E
    xf = synth.normal_f32((T, H), cfg.cid, 0, 7)
    g = torch.from_numpy(synth.normal_f32((T, E), cfg.cid, 1, 7)).to(dev)
    x = torch.from_numpy(xf).to(dev) if d["x"].dtype == torch.float32 \
        else bf16_dev(synth.f32_to_bf16_bits(xf), dev)
    return x, g


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _check_replays(call, x, g, x2, g2, out, other):
    """Eager results on both input sets, then a graph of `call` replayed four
    times, the inputs swapped in place between replays, with `other` (an
    eager layer call on buffers of its own) and synchronisations between."""
    x1, g1 = x.clone(), g.clone()
    call()                                    # also the first launch of every kernel
    torch.cuda.synchronize()
    ref1 = out.clone()
    x.copy_(x2)
    g.copy_(g2)
    call()
    torch.cuda.synchronize()
    ref2 = out.clone()
    assert not _same_bits(ref1, ref2)
    x.copy_(x1)
    g.copy_(g1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        assert _same_bits(out, ref1 if i % 2 == 0 else ref2), "replay %d" % i
        other()
        torch.cuda.synchronize()
        if i % 2 == 0:
            x.copy_(x2)
            g.copy_(g2)
        else:
            x.copy_(x1)
            g.copy_(g1)
        torch.cuda.synchronize()


@pytest.mark.parametrize("name,layout", [("tiny", "plain"), ("decode16", "packed"),
                                         ("prefill", "packed")])
def test_forward_graph_replays(moe, dev, name, layout):
    cfg = synth.CONFIGS[name]
    d = layer_inputs(cfg, dev)
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk
    w1, w2 = d["w1"], d["w2"]
    if layout == "packed":
        w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
    x, g = d["x"].clone(), d["gating"].clone()
    x2, g2 = _second_inputs(cfg, d, dev)
    ws = torch.empty(moe.moe_forward_workspace_size(T, H, I, E, K), dtype=torch.uint8, device=dev)
    ws_o = torch.empty_like(ws)
    out, out_o = torch.empty_like(x), torch.empty_like(x)
    kw = dict(num_expert_group=cfg.groups, topk_group=cfg.topk_group,
              renormalize=cfg.renormalize, routed_scaling_factor=cfg.scale)

    def call():
        moe.moe_forward(x, g, w1, w2, K, out=out, workspace=ws, **kw)

    def other():
        moe.moe_forward(x2, g2, w1, w2, K, out=out_o, workspace=ws_o, **kw)

    _check_replays(call, x, g, x2, g2, out, other)


def test_noalloc_graph_replays(moe, dev):
    """The call that allocates nothing, on the library's static scratch; the
    eager calls between replays use the same scratch (ordered on one
    stream, so they do not overlap)."""
    cfg = synth.CONFIGS["decode16"]
    d = layer_inputs(cfg, dev)
    w1, w2 = moe.moe_pack_weights(d["w1"], "silu_mul"), moe.moe_pack_weights(d["w2"], "none")
    x, g = d["x"].clone(), d["gating"].clone()
    x2, g2 = _second_inputs(cfg, d, dev)
    out, out_o = torch.empty_like(x), torch.empty_like(x)
    kw = dict(num_expert_group=cfg.groups, topk_group=cfg.topk_group,
              renormalize=cfg.renormalize, routed_scaling_factor=cfg.scale)

    def call():
        moe.moe_forward_noalloc(x, g, w1, w2, cfg.topk, out, **kw)

    def other():
        moe.moe_forward_noalloc(x2, g2, w1, w2, cfg.topk, out_o, **kw)

    _check_replays(call, x, g, x2, g2, out, other)


def test_w8a8_graph_replays(moe, dev):
    cfg = synth.CONFIGS["tiny"]
    d = layer_inputs(cfg, dev, x_dtype="bf16")
    T, H, I, E, K = cfg.T, cfg.H, cfg.I, cfg.E, cfg.topk
    w1q, s1 = oracle.quantize_weight_per_channel(d["w1_host"])   # input preparation
    w2q, s2 = oracle.quantize_weight_per_channel(d["w2_host"])
    W1 = moe.moe_pack_weights(torch.from_numpy(w1q).to(dev), "silu_mul")
    W2 = moe.moe_pack_weights(torch.from_numpy(w2q).to(dev), "none")
    S1 = torch.from_numpy(s1.astype(np.float32)).to(dev)
    S2 = torch.from_numpy(s2.astype(np.float32)).to(dev)
    x, g = d["x"].clone(), d["gating"].clone()
    x2, g2 = _second_inputs(cfg, d, dev)
    ws = torch.empty(moe.moe_forward_w8a8_workspace_size(T, H, I, E, K), dtype=torch.uint8,
                     device=dev)
    ws_o = torch.empty_like(ws)
    out, out_o = torch.empty_like(x), torch.empty_like(x)

    def call():
        moe.moe_forward_w8a8(x, g, W1, S1, W2, S2, K, out=out, workspace=ws)

    def other():
        moe.moe_forward_w8a8(x2, g2, W1, S1, W2, S2, K, out=out_o, workspace=ws_o)

    _check_replays(call, x, g, x2, g2, out, other)

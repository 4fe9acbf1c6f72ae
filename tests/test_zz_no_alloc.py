"""GPU check of moe_forward_noalloc, the layer call that allocates nothing
(its workspace is the library's static per-device scratch): through the C
ABI, two calls in a row (the second with fewer tokens) give bit-identical
results to moe_forward on a workspace of its own: bf16 tokens on packed
weights (the expert-wide tiles for the first call, 300 pairs per expert,
then the 256 x 64 tiles) and f32 tokens on plain weights; the first call is
also checked against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_host_f64, layer_inputs, require_gpu
from parity import BAR_BF16, max_abs_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


def _cfg(T, sub, x_dtype, **kw):
    from synth.configs import Config
    return Config(21, "noalloc", T=T, H=512, I=384, E=32, topk=4, x_dtype=x_dtype, w_std=0.05,
                  extra={"sub": sub}, **kw)


def _host(out):
    return out.cpu().numpy().astype(np.float64) if out.dtype == torch.float32 \
        else bf16_host_f64(out)


@pytest.mark.parametrize("x_dtype,layout,sizes", [("bf16", "packed", (2400, 100)),
                                                  ("bf16", "packed", (600, 100)),
                                                  ("f32", "plain", (600, 100))])
def test_noalloc_matches_moe_forward(moe, dev, x_dtype, layout, sizes):
    if x_dtype == "bf16" and sizes[0] == 2400:
        assert moe.moe_forward_block_m(2400, 32, 4, "bf16", "packed") == 32   # expert-wide
    for i, T in enumerate(sizes):               # the second call is smaller
        cfg = _cfg(T, i, x_dtype, groups=4, topk_group=2, scale=1.5)
        d = layer_inputs(cfg, dev)
        w1, w2 = d["w1"], d["w2"]
        if layout == "packed":
            w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
        args = (d["x"], d["gating"], w1, w2, cfg.topk)
        kw = dict(num_expert_group=cfg.groups, topk_group=cfg.topk_group,
                  routed_scaling_factor=cfg.scale)
        ids = torch.empty((T, cfg.topk), dtype=torch.int32, device=dev)
        wts = torch.empty((T, cfg.topk), dtype=torch.float32, device=dev)
        out = torch.full_like(d["x"], float("nan"))
        moe.moe_forward_noalloc(*args, out, topk_weights_out=wts, topk_ids_out=ids, **kw)
        ref = moe.moe_forward(*args, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "T=%d: differs from moe_forward" % T
        if i == 0:
            want = oracle.moe_layer_expert_loop(d["x_host"], d["w1_host"], d["w2_host"],
                                                wts.cpu().numpy().astype(np.float64),
                                                ids.cpu().numpy())
            err = max_abs_rel(_host(out), want)
            print("noalloc %s %s T=%d err=%.3e" % (x_dtype, layout, T, err))
            assert err <= BAR_BF16


def test_noalloc_rejects_oversized_layer(moe, dev):
    """A layer whose workspace exceeds the scratch is refused on the host."""
    T, H, I, E, K = 4096, 2048, 768, 128, 8
    assert moe.moe_forward_workspace_size(T, H, I, E, K) > moe.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    g = torch.zeros((T, E), dtype=torch.float32, device=dev)
    w1 = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=dev)
    w2 = torch.zeros((E, H, I), dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_noalloc(x, g, w1, w2, K, torch.empty_like(x))
    assert e.value.status == -5     # MOE_ERR_WORKSPACE

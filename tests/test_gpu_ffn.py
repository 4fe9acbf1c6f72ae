"""GPU checks of moe_grouped_ffn (both GEMMs in one persistent launch): its
h and y are bit-identical to two moe_grouped_gemm calls on the same
alignment (the same tiles and arithmetic), for every tile block size, both
weight layouts, a workspace that starts as garbage and repeated calls; at
the prefill size every pair row y and the summed output also meet the
oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bf16_host_f64, layer_inputs, require_gpu
from parity import BAR_BF16, check_routing, max_abs_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


def _two_launches(moe, x, w1, w2, K, s, e, tot, bm, w, P):
    h = torch.zeros((s.numel(), w1.shape[1] // 2), dtype=torch.bfloat16, device=x.device)
    moe.moe_grouped_gemm(x, w1, s, e, tot, bm, P, a_rows="pair", a_row_div=K,
                         epilogue="silu_mul", C=h, c_rows="sorted")
    y = moe.moe_grouped_gemm(h, w2, s, e, tot, bm, P, a_rows="sorted", topk_weights=w,
                             c_rows="pair")
    return h, y


def _valid_rows(s, tot, P):
    sn, total = s.cpu().numpy(), int(tot.cpu().numpy()[0])
    return np.flatnonzero((np.arange(sn.size) < total) & (sn < P))


def _compare(moe, d, cfg, bm, layout, ws=None):
    x, K, E = d["x"], cfg.topk, cfg.E
    w, ids = moe.moe_route(d["gating"], K, cfg.groups, cfg.topk_group, "softmax",
                           cfg.renormalize, cfg.scale)
    P = ids.numel()
    s, e, tot = moe.moe_align_block_size(ids, E, bm)
    w1, w2 = d["w1"], d["w2"]
    if layout == "packed":
        w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
    h_ref, y_ref = _two_launches(moe, x, w1, w2, K, s, e, tot, bm, w, P)
    if ws is None:
        ws = torch.empty(moe.moe_grouped_ffn_workspace_size(s.numel(), E, bm), dtype=torch.uint8,
                         device=x.device)
    h = torch.zeros_like(h_ref)
    h, y = moe.moe_grouped_ffn(x, w1, w2, K, s, e, tot, bm, w, h=h, workspace=ws)
    torch.cuda.synchronize()
    rows = torch.from_numpy(_valid_rows(s, tot, P)).to(x.device)
    assert torch.equal(h[rows], h_ref[rows])
    assert torch.equal(y, y_ref)
    # no wait of the launch ran into its spin limit
    assert moe.wait_flag(ws, moe.moe_grouped_ffn_wait_flag_offset(s.numel(), bm)) == 0
    return w, ids, y


def _cfg(T, H, I, E, K, sub=0, **kw):
    from synth.configs import Config
    return Config(13, "ffn", T=T, H=H, I=I, E=E, topk=K, x_dtype="bf16", w_std=0.05,
                  extra={"sub": sub}, **kw)


@pytest.mark.parametrize("bm", [64, 128, 256])
@pytest.mark.parametrize("layout", ["plain", "packed"])
def test_ffn_equals_two_launches(moe, dev, bm, layout):
    for cfg in (_cfg(64, 128, 256, 8, 2), _cfg(600, 256, 384, 16, 4, sub=1),
                _cfg(37, 192, 160, 40, 5, sub=2, groups=8, topk_group=3)):
        d = layer_inputs(cfg, dev)
        _compare(moe, d, cfg, bm, layout)


def test_ffn_garbage_and_reused_workspace(moe, dev):
    """Counters and expert table come from the set-up kernel, whatever the
    workspace held; a second call on the same workspace starts clean."""
    ws = torch.full((1 << 16,), 0x7f, dtype=torch.uint8, device=dev)
    for sub, T in enumerate([300, 41, 300]):
        cfg = _cfg(T, 256, 384, 16, 4, sub=sub)
        d = layer_inputs(cfg, dev)
        _compare(moe, d, cfg, 64, "packed", ws=ws)


def test_ffn_one_expert_many_blocks(moe, dev):
    """Every pair on one expert: the per-XCD block ranges split that expert."""
    cfg = _cfg(2000, 128, 256, 4, 1, sub=3)
    d = layer_inputs(cfg, dev)
    d["gating"] = torch.zeros_like(d["gating"])
    d["gating"][:, 2] = 10.0
    w, ids, _ = _compare(moe, d, cfg, 64, "packed")
    assert (ids.cpu().numpy() == 2).all()


@pytest.mark.timeout(600)
def test_ffn_prefill_matches_oracle(moe, dev):
    """The benchmark's launch (prefill layer, packed weights, block_m 128):
    bit-equal to the two-launch path, every one of its 32768 pair rows y
    within the bf16 bar of the oracle's pair terms, and their k-order sums
    within the bar of the oracle layer."""
    cfg = synth.CONFIGS["prefill"]
    d = layer_inputs(cfg, dev)
    w, ids, y = _compare(moe, d, cfg, 128, "packed")
    T, K, H = cfg.T, cfg.topk, cfg.H
    wn, idn = w.cpu().numpy().astype(np.float64), ids.cpu().numpy()
    # the oracle runs on the routing the GPU produced, which meets the
    # oracle's routing under the near-tie rule
    check_routing(wn, idn, d["gating_host"], K, True, 1, 1, "softmax", 1.0)
    ref = oracle.moe_layer_pair_rows(d["x_host"], d["w1_host"], d["w2_host"], wn, idn)
    err_y = max_abs_rel(bf16_host_f64(y).reshape(T, K, H), ref)
    out = y.view(T, K, H).float().sum(1)
    err = max_abs_rel(out.cpu().numpy().astype(np.float64), ref.sum(axis=1))
    print("ffn prefill, all pair rows: y err=%.3e, summed err=%.3e" % (err_y, err))
    assert err_y <= BAR_BF16 and err <= BAR_BF16


def test_ffn_wait_gives_up_at_spin_limit(moe, dev):
    """Failure handling, forced from the host: with a spin limit of one poll,
    down tiles that find their token block's gate_up tiles unfinished stop
    waiting and set the workspace flag, and every kernel still ends (h is
    then read early; the output is not checked).  With the default limit
    restored the same call on the same workspace is exact again and the flag
    reads 0.  Shape: few token blocks with 16 gate_up tiles each (K = 2048
    per tile), so all tiles are in flight at once and down tiles must wait."""
    cfg = _cfg(512, 2048, 2048, 8, 1, sub=6)
    d = layer_inputs(cfg, dev)
    bm = 64
    w, ids = moe.moe_route(d["gating"], 1)
    s, e, tot = moe.moe_align_block_size(ids, cfg.E, bm)
    ws = torch.empty(moe.moe_grouped_ffn_workspace_size(s.numel(), cfg.E, bm),
                     dtype=torch.uint8, device=dev)
    off = moe.moe_grouped_ffn_wait_flag_offset(s.numel(), bm)
    moe.moe_set_wait_spin_limit(1)
    try:
        moe.moe_grouped_ffn(d["x"], d["w1"], d["w2"], 1, s, e, tot, bm, w, workspace=ws)
        torch.cuda.synchronize()
        flagged = moe.wait_flag(ws, off)
    finally:
        moe.moe_set_wait_spin_limit(0)
    assert flagged == 1
    _compare(moe, d, cfg, bm, "plain", ws=ws)


def _sum_k_bf16(y, T, K):
    """Host sum of each token's K pair rows in k order, float32 from 0, then
    round to bf16 (the top-k reduce's arithmetic, written out)."""
    yf = y.float().cpu().view(T, K, -1)
    acc = torch.zeros_like(yf[:, 0])
    for k in range(K):
        acc += yf[:, k]
    return acc.to(torch.bfloat16)


@pytest.mark.parametrize("case", ["prefill", "decode16", "ragged64", "ragged128", "one_token"])
def test_forward_is_k_order_sum_of_ffn_rows(moe, dev, case):
    """moe_forward with bf16 x and block_m 64 / 128 (persistent launch, then the
    top-k reduce) is bit-identical to the pair rows of moe_grouped_ffn on the
    same routing and alignment, summed per token in k order in float32 and
    rounded to bf16 on the host: for both weight layouts, at the prefill and
    decode sizes, with H not a multiple of the 256-column tile, and with most
    experts empty (one token)."""
    if case in ("prefill", "decode16"):
        cfg = synth.CONFIGS[case]
    elif case == "one_token":
        cfg = _cfg(1, 4096, 512, 32, 8, sub=7)
    else:
        cfg = _cfg(333, 272, 160, 40, 6, sub=8 if case == "ragged64" else 9, groups=8,
                   topk_group=3)
    bm = 128 if case in ("prefill", "ragged128") else 64
    d = layer_inputs(cfg, dev)
    T, K, E = cfg.T, cfg.topk, cfg.E
    layouts = ["packed"] if case == "decode16" else ["plain", "packed"]
    for layout in layouts:
        w1, w2 = d["w1"], d["w2"]
        if layout == "packed":
            w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
        w, ids = moe.moe_route(d["gating"], K, cfg.groups, cfg.topk_group, "softmax",
                               cfg.renormalize, cfg.scale)
        s, e, tot = moe.moe_align_block_size(ids, E, bm)
        _, y = moe.moe_grouped_ffn(d["x"], w1, w2, K, s, e, tot, bm, w)
        ref = _sum_k_bf16(y, T, K)
        del y
        ws = torch.full((moe.moe_forward_workspace_size(T, cfg.H, cfg.I, E, K, bm),), 0x33,
                        dtype=torch.uint8, device=dev)
        ids2 = torch.empty_like(ids)
        out = moe.moe_forward(d["x"], d["gating"], w1, w2, K, cfg.groups, cfg.topk_group,
                              "softmax", cfg.renormalize, cfg.scale, block_m=bm,
                              topk_ids_out=ids2, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids2, ids)
        o = out.cpu()
        ndiff = int((o.view(torch.int16) != ref.view(torch.int16)).sum())
        print("%s %s block_m %d: %d of %d outputs differ" % (case, layout, bm, ndiff, o.numel()))
        assert ndiff == 0
        off = moe.moe_forward_wait_flag_offset(T, cfg.H, cfg.I, E, K, bm, "bf16", layout)
        assert moe.wait_flag(ws, off) == 0


@pytest.mark.parametrize("y_dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("bm", [64, 128])
def test_ffn_other_output_dtypes(moe, dev, y_dtype, bm):
    """y in float32 or float16 (the persistent launch's other down-tile
    epilogues): bit-identical to two moe_grouped_gemm launches writing the
    same dtype, on both weight layouts, with H not a multiple of 256."""
    cfg = _cfg(600, 272, 384, 16, 4, sub=10)
    d = layer_inputs(cfg, dev)
    K, E = cfg.topk, cfg.E
    w, ids = moe.moe_route(d["gating"], K)
    P = ids.numel()
    s, e, tot = moe.moe_align_block_size(ids, E, bm)
    for layout in ("plain", "packed"):
        w1, w2 = d["w1"], d["w2"]
        if layout == "packed":
            w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
        h = torch.zeros((s.numel(), cfg.I), dtype=torch.bfloat16, device=dev)
        moe.moe_grouped_gemm(d["x"], w1, s, e, tot, bm, P, a_rows="pair", a_row_div=K,
                             epilogue="silu_mul", C=h, c_rows="sorted")
        y_ref = moe.moe_grouped_gemm(h, w2, s, e, tot, bm, P, a_rows="sorted", topk_weights=w,
                                     c_dtype=y_dtype, c_rows="pair")
        ws = torch.empty(moe.moe_grouped_ffn_workspace_size(s.numel(), E, bm), dtype=torch.uint8,
                         device=dev)
        _, y = moe.moe_grouped_ffn(d["x"], w1, w2, K, s, e, tot, bm, w, y_dtype=y_dtype,
                                   workspace=ws)
        torch.cuda.synchronize()
        assert y.dtype == y_dtype
        assert torch.equal(y, y_ref), layout
        assert moe.wait_flag(ws, moe.moe_grouped_ffn_wait_flag_offset(s.numel(), bm)) == 0

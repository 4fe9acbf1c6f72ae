"""GPU checks of the layer's two GEMMs and its top-k reduce: at the prefill
size the per-pair rows y of gate_up (SiLU*up into h, sorted order) followed
by down (times the routing weight, pair order) meet the oracle's pair terms
on every row; moe_forward's output, on the tile kernels and on the
expert-wide tiles, is bit-identical to those rows summed per token in k
order on the host, on both weight layouts and several shapes."""

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


def _gemm_pair(moe, x, w1, w2, K, s, e, tot, bm, w, P, y_dtype=None):
    """gate_up into h (sorted rows), then down into y (pair rows)."""
    h = torch.zeros((s.numel(), w1.shape[1] // 2), dtype=torch.bfloat16, device=x.device)
    moe.moe_grouped_gemm(x, w1, s, e, tot, bm, P, a_rows="pair", a_row_div=K,
                         epilogue="silu_mul", C=h, c_rows="sorted")
    kw = {} if y_dtype is None else dict(c_dtype=y_dtype)
    y = moe.moe_grouped_gemm(h, w2, s, e, tot, bm, P, a_rows="sorted", topk_weights=w,
                             c_rows="pair", **kw)
    return h, y


def _cfg(T, H, I, E, K, sub=0, **kw):
    from synth.configs import Config
    return Config(13, "ffn", T=T, H=H, I=I, E=E, topk=K, x_dtype="bf16", w_std=0.05,
                  extra={"sub": sub}, **kw)


@pytest.mark.timeout(600)
def test_gemm_pair_prefill_matches_oracle(moe, dev):
    """The benchmark's configuration (prefill layer, packed weights, block_m
    128): every one of the 32768 pair rows y within the bf16 bar of the
    oracle's pair terms, and their k-order sums within the bar of the oracle
    layer."""
    cfg = synth.CONFIGS["prefill"]
    d = layer_inputs(cfg, dev)
    T, K, H, E = cfg.T, cfg.topk, cfg.H, cfg.E
    w1, w2 = moe.moe_pack_weights(d["w1"], "silu_mul"), moe.moe_pack_weights(d["w2"], "none")
    w, ids = moe.moe_route(d["gating"], K)
    s, e, tot = moe.moe_align_block_size(ids, E, 128)
    _, y = _gemm_pair(moe, d["x"], w1, w2, K, s, e, tot, 128, w, T * K)
    torch.cuda.synchronize()
    wn, idn = w.cpu().numpy().astype(np.float64), ids.cpu().numpy()
    # the oracle runs on the routing the GPU produced, which meets the
    # oracle's routing under the near-tie rule
    check_routing(wn, idn, d["gating_host"], K, True, 1, 1, "softmax", 1.0)
    ref = oracle.moe_layer_pair_rows(d["x_host"], d["w1_host"], d["w2_host"], wn, idn)
    err_y = max_abs_rel(bf16_host_f64(y).reshape(T, K, H), ref)
    out = y.view(T, K, H).float().sum(1)
    err = max_abs_rel(out.cpu().numpy().astype(np.float64), ref.sum(axis=1))
    print("gemm pair prefill, all pair rows: y err=%.3e, summed err=%.3e" % (err_y, err))
    assert err_y <= BAR_BF16 and err <= BAR_BF16


def _sum_k_bf16(y, T, K):
    """Host sum of each token's K pair rows in k order, float32 from 0, then
    round to bf16 (the top-k reduce's arithmetic, written out)."""
    yf = y.float().cpu().view(T, K, -1)
    acc = torch.zeros_like(yf[:, 0])
    for k in range(K):
        acc += yf[:, k]
    return acc.to(torch.bfloat16)


@pytest.mark.parametrize("case", ["prefill", "decode16", "ragged64", "ragged128", "one_token"])
def test_forward_is_k_order_sum_of_gemm_rows(moe, dev, case):
    """moe_forward with bf16 x and block_m 64 / 128 is bit-identical to the
    pair rows of the two GEMM launches on the same routing and alignment,
    summed per token in k order in float32 and rounded to bf16 on the host:
    for both weight layouts, at the prefill and decode sizes, with H not a
    multiple of the 256-column tile, and with most experts empty (one
    token).  moe_forward on the expert-wide tiles (block_m 32) gives the
    same bits: it runs the same MFMA sequence over K on other tiles (up to
    320 rows of one expert; partial K stages, partial column tiles, experts
    split over two tiles at the prefill size).  The workspace starts full
    of garbage."""
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
        _, y = _gemm_pair(moe, d["x"], w1, w2, K, s, e, tot, bm, w, T * K)
        ref = _sum_k_bf16(y, T, K)
        del y
        for fbm in (bm, 32):
            ws = torch.full((moe.moe_forward_workspace_size(T, cfg.H, cfg.I, E, K, fbm),), 0x33,
                            dtype=torch.uint8, device=dev)
            ids2 = torch.empty_like(ids)
            out = moe.moe_forward(d["x"], d["gating"], w1, w2, K, cfg.groups, cfg.topk_group,
                                  "softmax", cfg.renormalize, cfg.scale, block_m=fbm,
                                  topk_ids_out=ids2, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(ids2, ids)
            o = out.cpu()
            ndiff = int((o.view(torch.int16) != ref.view(torch.int16)).sum())
            print("%s %s forward block_m %d (rows at %d): %d of %d outputs differ"
                  % (case, layout, fbm, bm, ndiff, o.numel()))
            assert ndiff == 0
            del ws


@pytest.mark.parametrize("y_dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("bm", [64, 128])
def test_gemm_pair_other_output_dtypes(moe, dev, y_dtype, bm):
    """y in float32 or float16 (the down GEMM's other epilogues), on both
    weight layouts with H not a multiple of 256: within the bf16 bar of the
    oracle's pair terms, and the packed and plain layouts give identical
    bits."""
    cfg = _cfg(600, 272, 384, 16, 4, sub=10)
    d = layer_inputs(cfg, dev)
    T, K, E, H = cfg.T, cfg.topk, cfg.E, cfg.H
    w, ids = moe.moe_route(d["gating"], K)
    P = ids.numel()
    s, e, tot = moe.moe_align_block_size(ids, E, bm)
    ref = oracle.moe_layer_pair_rows(d["x_host"], d["w1_host"], d["w2_host"],
                                     w.cpu().numpy().astype(np.float64), ids.cpu().numpy())
    ys = []
    for layout in ("plain", "packed"):
        w1, w2 = d["w1"], d["w2"]
        if layout == "packed":
            w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
        _, y = _gemm_pair(moe, d["x"], w1, w2, K, s, e, tot, bm, w, P, y_dtype=y_dtype)
        torch.cuda.synchronize()
        assert y.dtype == y_dtype
        err = max_abs_rel(y.double().cpu().numpy().reshape(T, K, H), ref)
        print("y %s block_m %d %s err=%.3e" % (y_dtype, bm, layout, err))
        assert err <= BAR_BF16
        ys.append(y)
    assert torch.equal(ys[0], ys[1])


def _check_tile_table(table, eids, total, E):
    """The tile table partitions every expert's blocks into ceil(n / 10)
    runs of consecutive blocks whose sizes differ by at most one."""
    t = table.cpu().numpy()
    ex = eids.cpu().numpy()
    nblk = int(total.cpu().numpy()[0]) // 32
    n = int(t[0])
    tiles = t[1:1 + 3 * n].reshape(n, 3)
    seen = np.zeros(nblk, dtype=np.int64)
    per_expert = {}
    for e, b0, nb in tiles:
        assert 1 <= nb <= 10 and 0 <= b0 and b0 + nb <= nblk
        assert (ex[b0:b0 + nb] == e).all()
        seen[b0:b0 + nb] += 1
        per_expert.setdefault(int(e), []).append(int(nb))
    assert (seen == 1).all()
    for e, sizes in per_expert.items():
        cnt = int((ex[:nblk] == e).sum())
        assert len(sizes) == -(-cnt // 10) and max(sizes) - min(sizes) <= 1
    assert len(per_expert) == len(np.unique(ex[:nblk]))


def _by_pair(h, s, P):
    """Rows of h (sorted order) keyed by pair index."""
    sn = s.cpu().numpy()
    pos = np.nonzero((sn >= 0) & (sn < P))[0]
    out = torch.empty((P, h.shape[1]), dtype=h.dtype)
    out[torch.from_numpy(sn[pos]).long()] = h.cpu()[torch.from_numpy(pos).long()]
    return out


@pytest.mark.parametrize("case", ["prefill", "decode16", "ragged", "one_token", "big_expert"])
def test_wide_gemms_match_tile_gemms(moe, dev, case):
    """moe_grouped_gemm_wide (gate_up with SiLU*up, then down with the
    routing weight) on a block-32 alignment gives the same h (per pair) and
    the same y bits as moe_grouped_gemm on the 256 x 128 / 256 x 64 tiles,
    on both weight layouts: at the prefill and decode sizes, with H and I
    not multiples of the tiles (partial K stages, partial column tiles),
    with most experts empty, and with one expert of 700 pairs (three
    tiles).  The tile table is checked on the host."""
    if case in ("prefill", "decode16"):
        cfg = synth.CONFIGS[case]
    elif case == "one_token":
        cfg = _cfg(1, 4096, 512, 32, 8, sub=11)
    elif case == "big_expert":
        cfg = _cfg(700, 256, 384, 8, 1, sub=12)
    else:
        cfg = _cfg(333, 272, 160, 40, 6, sub=13, groups=8, topk_group=3)
    d = layer_inputs(cfg, dev)
    T, K, E = cfg.T, cfg.topk, cfg.E
    P = T * K
    g = d["gating"]
    if case == "big_expert":   # every token's best expert is expert 5
        g = g.clone()
        g[:, 5] += 8.0
    w, ids = moe.moe_route(g, K, cfg.groups, cfg.topk_group, "softmax", cfg.renormalize,
                           cfg.scale)
    bm = 128 if case == "prefill" else 64
    s, e, tot = moe.moe_align_block_size(ids, E, bm)
    s32, e32, tot32 = moe.moe_align_block_size(ids, E, 32)
    table = moe.moe_wide_tile_table(e32, tot32, E, s32.numel())
    torch.cuda.synchronize()
    _check_tile_table(table, e32, tot32, E)
    layouts = ["packed"] if case == "decode16" else ["plain", "packed"]
    for layout in layouts:
        w1, w2 = d["w1"], d["w2"]
        if layout == "packed":
            w1, w2 = moe.moe_pack_weights(w1, "silu_mul"), moe.moe_pack_weights(w2, "none")
        h, y = _gemm_pair(moe, d["x"], w1, w2, K, s, e, tot, bm, w, P)
        hw = torch.zeros((s32.numel(), cfg.I), dtype=torch.bfloat16, device=dev)
        moe.moe_grouped_gemm_wide(d["x"], w1, s32, e32, tot32, table, P, a_rows="pair",
                                  a_row_div=K, epilogue="silu_mul", C=hw, c_rows="sorted")
        yw = moe.moe_grouped_gemm_wide(hw, w2, s32, e32, tot32, table, P, a_rows="sorted",
                                       topk_weights=w, c_rows="pair")
        torch.cuda.synchronize()
        hp, hwp = _by_pair(h, s, P), _by_pair(hw, s32, P)
        nh = int((hp.view(torch.int16) != hwp.view(torch.int16)).sum())
        ny = int((y.cpu().view(torch.int16) != yw.cpu().view(torch.int16)).sum())
        print("%s %s: h differs in %d, y in %d of %d" % (case, layout, nh, ny, y.numel()))
        assert nh == 0 and ny == 0
        del h, y, hw, yw

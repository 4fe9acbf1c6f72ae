"""GPU parity of gmm_int8 against the oracle's dequantised result (exact
integer sums times both scales).  Bar: max-abs-rel 3e-2 (the fp16 output
rounding alone is ~5e-4)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import gmm_inputs, require_gpu
from parity import BAR_INT8, max_abs_rel

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


def _run_and_check(moe, dev, M, K, N, E, sizes, seed, bar=BAR_INT8, layout="plain"):
    h, d = gmm_inputs(M, K, N, E, sizes, seed, dev)
    Y = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev)
    W = moe.moe_pack_weights(d["wq"]) if layout == "packed" else d["wq"]
    moe.gmm_int8(d["xq"], W, d["sx"], d["sw"], d["off"], output=Y)
    torch.cuda.synchronize()
    got = Y.float().cpu().numpy()
    ref = oracle.gmm_int8(h["xq"], h["wq"], h["sx"], h["sw"], h["off"])
    assert np.isfinite(got).all()
    err = max_abs_rel(got, ref)
    assert err <= bar, err
    return got, ref, h, err


@pytest.mark.parametrize("layout", ["plain", "packed"])
def test_int8_workload_zipf(moe, dev, layout):
    cfg = synth.CONFIGS["int8gmm"]
    sizes = synth.zipf_group_sizes(cfg.T, cfg.E, cfg.extra["zipf_s"], cfg.cid, 9)
    assert (sizes == 0).any() and (sizes == 1).any()
    got, ref, h, err = _run_and_check(moe, dev, cfg.T, cfg.H, cfg.I, cfg.E, sizes, cfg.cid,
                                      layout=layout)
    print("int8 gmm workload (%s weights) err=%.3e" % (layout, err))


@pytest.mark.parametrize("sizes", [
    [0, 0, 5, 0, 123, 1, 0],          # empty first/last experts, single row
    [300],                            # one expert, several full tiles + tail
    [1] * 9,                          # one row each
    [128, 128, 0, 256],               # exact tile multiples
    [0, 0, 0, 1]])
@pytest.mark.parametrize("layout", ["plain", "packed"])
def test_int8_edge_groups(moe, dev, sizes, layout):
    E = len(sizes)
    _run_and_check(moe, dev, int(np.sum(sizes)), 256, 192, E, sizes, 50 + E, layout=layout)


@pytest.mark.parametrize("layout", ["plain", "packed"])
def test_int8_more_tiles_than_one_round(moe, dev, layout):
    """About 600 tiles of 256 x 128, more than one round of resident
    workgroups: every output is written once and matches the oracle."""
    rng = np.random.default_rng(77)
    sizes = rng.integers(0, 500, size=40)
    sizes[[3, 17]] = 0
    sizes[5] = 1
    M = int(sizes.sum())
    _run_and_check(moe, dev, M, 64, 2048, 40, sizes, 78, layout=layout)


@pytest.mark.parametrize("layout", ["plain", "packed"])
def test_int8_small_dims(moe, dev, layout):
    _run_and_check(moe, dev, 40, 16, 16, 3, [10, 20, 10], 61, layout=layout)
    _run_and_check(moe, dev, 70, 144, 48, 2, [33, 37], 62, layout=layout)   # K tail, N < 128
    _run_and_check(moe, dev, 90, 80, 272, 2, [60, 30], 65, layout=layout)   # N past one tile


def test_int8_empty(moe, dev):
    h, d = gmm_inputs(0, 64, 32, 2, [0, 0], 63, dev)
    Y = moe.gmm_int8(d["xq"], d["wq"], d["sx"], d["sw"], d["off"])
    torch.cuda.synchronize()
    assert Y.shape == (0, 32)


def test_int8_quantisation_error_informational(moe, dev):
    """Not gated beyond the bar: error of the int8 GMM against the float32
    GEMM of the unquantised operands, as the article's quality check does."""
    sizes = [40, 0, 88]
    got, ref, h, _ = _run_and_check(moe, dev, 128, 512, 256, 3, sizes, 64)
    fp = oracle.gmm(h["x"].astype(np.float64),
                    np.stack([h["w_f32"][e] for e in range(3)]).astype(np.float64), h["off"])
    rel = max_abs_rel(got, fp)
    cos = float((got * fp).sum() / np.sqrt((got * got).sum() * (fp * fp).sum()))
    print("int8 vs fp32 GEMM: max-abs-rel %.3e cosine %.6f" % (rel, cos))
    assert cos > 0.99


@pytest.mark.parametrize("mtiles,N", [
    (65, 2048),    # one n-tile of each expert per XCD: 65 tiles each, one past a round
    (97, 2048),
    (40, 4096)])   # two n-tiles of each expert per XCD
def test_int8_tile_order_shapes(moe, dev, mtiles, N):
    """Tiles dealt to the XCDs by expert size (ties by id): experts of 1 to
    128 rows, many of equal size, every output written once."""
    rng = np.random.default_rng(mtiles * 1000 + N)
    sizes = rng.integers(1, 129, size=mtiles)
    sizes[::7] = 128
    sizes[::11] = 5
    _run_and_check(moe, dev, int(sizes.sum()), 128, N, mtiles, sizes, 90 + mtiles,
                   layout="packed")


def test_int8_tile_order_narrow_n(moe, dev):
    """N = 256 (one n-tile per expert): the experts themselves are dealt to
    the XCDs in turn, so the XCDs hold different numbers of tiles."""
    sizes = np.full(600, 3)
    sizes[::5] = 250
    sizes[::9] = 0
    _run_and_check(moe, dev, int(sizes.sum()), 64, 256, 600, sizes, 95, layout="packed")

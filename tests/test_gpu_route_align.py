"""GPU parity of moe_route and moe_align_block_size against the oracle
(called through the C ABI).  Ids and alignment metadata must be bit-exact
(routing ids: up to the near-tie rule), routing weights within 1e-5."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import require_gpu
from parity import check_routing

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


def _route(moe, logits_np, topk, renorm, G, Kg, scoring, scale, dev):
    g = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).to(dev)
    w, ids = moe.moe_route(g, topk, G, Kg, scoring, renorm, scale)
    torch.cuda.synchronize()
    return w.cpu().numpy(), ids.cpu().numpy()


def _check(moe, logits, topk, renorm, G, Kg, scoring, scale, dev, allow_ties=False):
    w, ids = _route(moe, logits, topk, renorm, G, Kg, scoring, scale, dev)
    exact, ties, err = check_routing(w, ids, logits.astype(np.float32).astype(np.float64),
                                     topk, renorm, G, Kg, scoring, scale)
    if not allow_ties:
        assert ties == 0, "unexpected near-tie rows on random data"
    return exact, ties, err


# ---- the routing workload and its variants --------------------------------

@pytest.mark.parametrize("scoring,renorm,scale", [
    ("softmax", True, 1.0), ("softmax", False, 1.0), ("softmax", True, 2.5),
    ("sigmoid", True, 1.0), ("sigmoid", False, 2.5)])
def test_route_grouped_workload(moe, dev, scoring, renorm, scale):
    logits = synth.normal_f32((83, 256), 2, 0)
    _check(moe, logits, 8, renorm, 8, 4, scoring, scale, dev)


@pytest.mark.parametrize("T,E,K,G,Kg", [
    (64, 8, 2, 1, 1), (4096, 128, 8, 1, 1), (16, 256, 8, 8, 4), (64, 256, 8, 8, 4),
    (7, 96, 6, 4, 2), (5, 100, 3, 1, 1), (3, 1024, 64, 1, 1), (2, 1024, 8, 32, 2),
    (1, 64, 64, 1, 1), (33, 40, 5, 8, 8), (9, 64, 1, 64, 1), (300, 512, 16, 16, 3)])
def test_route_shapes(moe, dev, T, E, K, G, Kg):
    logits = synth.normal_f32((T, E), 2, 100 + E, T)
    _check(moe, logits, K, True, G, Kg, "softmax", 1.0, dev)


def test_route_gtk_worked_example(moe, dev, golden_dir):
    with open(os.path.join(golden_dir, "gtk_worked_example.json")) as f:
        g = json.load(f)
    logits = np.log(np.array(g["scores"], dtype=np.float64))[None].astype(np.float32)
    w, ids = _route(moe, logits, g["topk"], True, g["num_expert_group"], g["topk_group"],
                    "softmax", 1.0, dev)
    assert ids[0].tolist() == g["ids"]
    np.testing.assert_allclose(w[0], [0.9 / 1.7, 0.8 / 1.7], rtol=2e-6)


def test_route_msg_seeded_example(moe, dev, golden_dir):
    with open(os.path.join(golden_dir, "msg_seeded_example.json")) as f:
        g = json.load(f)
    torch.manual_seed(0)
    _x, gating = torch.randn(g["T"], g["H"]), torch.randn(g["T"], g["E"])
    w, ids = _route(moe, gating.numpy(), g["topk"], True, 1, 1, "softmax", 1.0, dev)
    assert ids.tolist() == g["ids"]
    np.testing.assert_allclose(np.round(w, 3), g["weights_3dp"], atol=1e-9)


def test_route_ties_lowest_index(moe, dev):
    # few distinct values: exact ties at expert and group level, on purpose
    rng = np.random.default_rng(5)
    logits = (rng.integers(-2, 3, size=(200, 64)) * 0.5).astype(np.float32)
    for (G, Kg, K) in [(1, 1, 8), (8, 3, 6), (4, 4, 16), (64, 5, 5)]:
        w, ids = _route(moe, logits, K, True, G, Kg, "softmax", 1.0, dev)
        _, ref = oracle.grouped_topk(logits.astype(np.float64), K, True, G, Kg)
        assert (ids == ref).all(), (G, Kg, K)


def test_route_all_equal_and_signed_zero(moe, dev):
    logits = np.zeros((4, 32), np.float32)
    logits[1, ::2] = -0.0
    logits[2] = -0.0
    w, ids = _route(moe, logits, 4, True, 4, 2, "softmax", 1.0, dev)
    assert (ids == np.array([0, 1, 2, 3])).all()
    np.testing.assert_allclose(w, 0.25, rtol=1e-7)


def test_route_neg_inf(moe, dev):
    logits = synth.normal_f32((10, 64), 2, 7)
    logits[:, ::3] = -np.inf
    _check(moe, logits, 8, True, 4, 2, "softmax", 1.0, dev)
    _check(moe, logits, 8, False, 1, 1, "softmax", 1.0, dev)


def test_route_extremes(moe, dev):
    logits = synth.normal_f32((50, 128), 2, 8) * 30.0
    _check(moe, logits, 8, True, 8, 4, "softmax", 2.5, dev)
    # sigmoid saturates in fp64 for large logits: near-ties are allowed there
    _check(moe, logits, 8, True, 8, 4, "sigmoid", 1.0, dev, allow_ties=True)


def test_route_empty(moe, dev):
    g = torch.empty((0, 64), dtype=torch.float32, device=dev)
    w, ids = moe.moe_route(g, 4)
    torch.cuda.synchronize()
    assert w.shape == (0, 4)


# ---- alignment ------------------------------------------------------------

def _align_gpu(moe, ids_np, E, B, dev, ws=False):
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(dev)
    wsb = None
    if ws:   # the two-kernel path; the buffers start as garbage on purpose
        wsb = torch.full((moe.moe_align_workspace_size(ids.numel(), E),), 0x5a, dtype=torch.uint8,
                         device=dev)
    s, e, tot = moe.moe_align_block_size(ids, E, B, workspace=wsb)
    torch.cuda.synchronize()
    return s.cpu().numpy(), e.cpu().numpy(), int(tot.cpu().numpy()[0])


def _check_align(moe, ids_np, E, B, dev):
    """Both alignment paths (workspace-free and two-kernel) against the oracle."""
    rs, re_, rtotal = oracle.moe_align_block_size(ids_np, E, B)
    P = np.asarray(ids_np).size
    for ws in (False, True):
        s, e, total = _align_gpu(moe, ids_np, E, B, dev, ws)
        assert total == rtotal, ws
        assert (s[:total] == rs).all(), ws
        assert (e[:total // B] == re_).all(), ws
        assert (s[total:] == P).all(), ws
        assert (e[total // B:] == -1).all(), ws
        assert s.size == moe.moe_align_max_padded(P, E, B)


def test_align_msg_printout(moe, dev, golden_dir):
    with open(os.path.join(golden_dir, "msg_seeded_example.json")) as f:
        g = json.load(f)
    s, e, total = _align_gpu(moe, np.array(g["ids"]), g["E"], g["block_m"], dev)
    assert s[:total].tolist() == g["sorted_ids"]
    assert e[:total // g["block_m"]].tolist() == g["expert_ids"]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("B", [1, 4, 16, 32, 64, 128])
def test_align_random(moe, dev, seed, B):
    rng = np.random.default_rng(seed * 31 + B)
    E = int(rng.integers(1, 300))
    T = int(rng.integers(1, 700))
    K = int(rng.integers(1, min(E, 8) + 1))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    _check_align(moe, ids, E, B, dev)


@pytest.mark.parametrize("T,E,K,B", [(4096, 128, 8, 128), (4096, 128, 8, 64), (16, 256, 8, 16),
                                     (64, 256, 8, 16), (64, 8, 2, 32), (3000, 1024, 8, 16)])
def test_align_workload_shapes(moe, dev, T, E, K, B):
    logits = synth.normal_f32((T, E), 2, 200 + E, T)
    _, ids = oracle.grouped_topk(logits.astype(np.float64), K, True, 1, 1)
    _check_align(moe, ids, E, B, dev)


@pytest.mark.parametrize("P,E,B", [(32768, 128, 256),     # prefill pairs, block 256
                                   (100000, 128, 64),     # ids not cached in LDS
                                   (600000, 128, 128)])   # single-workgroup kernel
def test_align_large(moe, dev, P, E, B):
    """The three alignment kernels the library picks by size all agree with
    the oracle bit for bit."""
    rng = np.random.default_rng(P + E + B)
    ids = rng.integers(0, E, size=P).astype(np.int32)
    ids[: P // 7] = E // 3                     # one heavy expert
    _check_align(moe, ids, E, B, dev)


def test_align_skewed_and_edge(moe, dev):
    _check_align(moe, np.zeros(5000, np.int32), 64, 128, dev)          # one expert
    _check_align(moe, np.full(777, 63, np.int32), 64, 16, dev)         # last expert
    _check_align(moe, np.arange(1024, dtype=np.int32), 1024, 32, dev)  # one pair each
    _check_align(moe, np.zeros(0, np.int32), 16, 16, dev)              # no pairs
    _check_align(moe, np.array([0, 0, 0], np.int32), 1, 1, dev)        # E = 1, B = 1

"""GPU parity of moe_grouped_gemm (both kernels: weight-streaming for
block_m 16/32, MFMA tile for 64/128) against the oracle's sorted grouped
GEMM.  The sorted metadata handed to both sides comes from the oracle."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import bf16_dev, require_gpu
from parity import max_abs_rel

pytestmark = pytest.mark.gpu

BLOCKS = [16, 32, 64, 128, 256]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def moe(dev):
    import moe_grouped_topk_amd as m
    return m


def _meta(moe, ids, E, B, dev):
    """Oracle alignment, laid out in device buffers of the library's size."""
    s, e, total = oracle.moe_align_block_size(ids, E, B)
    P = np.asarray(ids).size
    cap = moe.moe_align_max_padded(P, E, B)
    sb = np.full(cap, P, np.int32)
    sb[:total] = s
    eb = np.full(cap // B, -1, np.int32)
    eb[:total // B] = e
    return (torch.from_numpy(sb).to(dev), torch.from_numpy(eb).to(dev),
            torch.tensor([total], dtype=torch.int32, device=dev), s, e, total)


def _tol(c_dtype):
    return 1e-5 if c_dtype == torch.float32 else 8e-3


def test_p1_worked_example(moe, dev, golden_dir):
    """[P1] 03.3 example embedded in the kernel's alignment: K padded from 3
    to 8 and N from 2 to 16 with zeros (the extra columns stay zero)."""
    with open(os.path.join(golden_dir, "p1_worked_example.json")) as f:
        g = json.load(f)
    x = np.zeros((2, 8), np.float32)
    x[:, :3] = g["x"]
    W = np.zeros((4, 16, 8), np.float32)
    for e, v in enumerate(g["expert_fill"]):
        W[e, :2, :3] = v
    ids = np.array(g["topk_ids"])
    for B in BLOCKS:
        sb, eb, tot, *_ = _meta(moe, ids, 4, B, dev)
        C = moe.moe_grouped_gemm(
            bf16_dev(synth.f32_to_bf16_bits(x), dev), bf16_dev(synth.f32_to_bf16_bits(W), dev),
            sb, eb, tot, B, 4, a_rows="pair", a_row_div=2, c_dtype=torch.float32)
        torch.cuda.synchronize()
        out = C.cpu().numpy()
        assert out[:, :2].reshape(2, 2, 2).tolist() == g["output"], B
        assert (out[:, 2:] == 0).all()


def _rand_case(seed, T, E, K_top, H, N, a_f32=False):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:K_top] for _ in range(T)])
    A = synth.normal_f32((T, H), 9, 0, seed)
    Bw = synth.normal_f32((E, N, H), 9, 1, seed, 0.05)
    wts = rng.random(T * K_top).astype(np.float32)
    return ids, A, Bw, wts


@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("epilogue", ["none", "silu_mul"])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_gemm_pair_rows(moe, dev, B, epilogue, c_dtype):
    T, E, Kt, H, N = 97, 7, 3, 136, 96        # K tail (136 = 2 stages + 8), N not /128
    ids, A, Bw, wts = _rand_case(B + (epilogue == "none"), T, E, Kt, H, N)
    Ab, Bb = synth.f32_to_bf16_bits(A), synth.f32_to_bf16_bits(Bw)
    sb, eb, tot, s, e, total = _meta(moe, ids, E, B, dev)
    P = ids.size
    w_dev = torch.from_numpy(wts).to(dev)
    C = torch.full((P, N // 2 if epilogue == "silu_mul" else N), float("nan"),
                   dtype=c_dtype, device=dev)
    moe.moe_grouped_gemm(bf16_dev(Ab, dev), bf16_dev(Bb, dev), sb, eb, tot, B, P,
                         a_rows="pair", a_row_div=Kt, topk_weights=w_dev, epilogue=epilogue,
                         C=C, c_rows="pair")
    torch.cuda.synchronize()
    A64, B64 = oracle.bf16_bits_to_f64(Ab), oracle.bf16_bits_to_f64(Bb)
    if epilogue == "none":
        ref, written = oracle.grouped_gemm_sorted(A64, B64, s, e, B, P, Kt, wts.astype(np.float64))
    else:
        gu, written = oracle.grouped_gemm_sorted(A64, B64, s, e, B, P, Kt)
        ref = oracle.silu_and_mul(gu) * wts.astype(np.float64)[:, None]
    assert written.all()
    got = C.float().cpu().numpy()
    assert np.isfinite(got).all()
    assert max_abs_rel(got, ref) <= _tol(c_dtype)


@pytest.mark.parametrize("B", [b for b in BLOCKS if b != 256])
def test_gemm_sorted_rows_and_f32_input(moe, dev, B):
    """A rows by sorted position (how the layer feeds its second GEMM), C rows
    by sorted position; float32 A rounded to bf16 on load."""
    T, E, Kt, H, N = 50, 5, 2, 64, 48
    ids, A, Bw, _ = _rand_case(77 + B, T, E, Kt, H, N)
    sb, eb, tot, s, e, total = _meta(moe, ids, E, B, dev)
    cap = sb.numel()
    As = synth.normal_f32((cap, H), 9, 5, B)            # one row per sorted position
    Bb = synth.f32_to_bf16_bits(Bw)
    C = torch.full((cap, N), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_grouped_gemm(torch.from_numpy(As).to(dev), bf16_dev(Bb, dev), sb, eb, tot, B,
                         ids.size, a_rows="sorted", C=C, c_rows="sorted")
    torch.cuda.synchronize()
    got = C.cpu().numpy()
    A_r = oracle.bf16_bits_to_f64(synth.f32_to_bf16_bits(As))   # the kernel's rounding point
    B64 = oracle.bf16_bits_to_f64(Bb)
    for pos in range(total):
        p = s[pos]
        if p >= ids.size:
            assert np.isnan(got[pos]).all()        # placeholder rows untouched
            continue
        ref = A_r[pos] @ B64[e[pos // B]].T
        assert max_abs_rel(got[pos], ref) <= 1e-5 * 4
    assert np.isnan(got[total:]).all()


@pytest.mark.parametrize("B", BLOCKS)
def test_gemm_skewed_experts(moe, dev, B):
    """One expert holds most pairs (many full blocks), others one pair or
    none: exercises full, partial and single-row blocks."""
    T, E, Kt, H, N = 300, 16, 1, 256, 128
    ids = np.zeros((T, 1), np.int64)
    ids[::37, 0] = 3
    ids[5, 0] = 15
    A = synth.normal_f32((T, H), 9, 7)
    Bw = synth.normal_f32((E, N, H), 9, 8, 0, 0.05)
    Ab, Bb = synth.f32_to_bf16_bits(A), synth.f32_to_bf16_bits(Bw)
    sb, eb, tot, s, e, total = _meta(moe, ids, E, B, dev)
    C = moe.moe_grouped_gemm(bf16_dev(Ab, dev), bf16_dev(Bb, dev), sb, eb, tot, B, T,
                             c_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_gemm_sorted(oracle.bf16_bits_to_f64(Ab), oracle.bf16_bits_to_f64(Bb),
                                        s, e, B, T, 1)
    assert max_abs_rel(C.cpu().numpy(), ref) <= 1e-5


def test_gemm_f32_input_rejected_at_256(moe, dev):
    ids = np.zeros((8, 1), np.int64)
    sb, eb, tot, *_ = _meta(moe, ids, 1, 256, dev)
    A = torch.zeros((8, 64), dtype=torch.float32, device=dev)
    Bw = torch.zeros((1, 32, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_gemm(A, Bw, sb, eb, tot, 256, 8)

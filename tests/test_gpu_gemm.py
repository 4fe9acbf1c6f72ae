"""GPU parity of moe_grouped_gemm (both kernels: weight-streaming for
block_m 16/32, MFMA tile for 64/128/256, plain and packed weights) against
the oracle's sorted grouped GEMM.  The sorted metadata handed to both sides
comes from the oracle."""

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


def _weights(moe, Bb, dev, layout, epilogue):
    """bf16 bits [E, N, K] -> device weights in the requested layout."""
    w = bf16_dev(Bb, dev)
    return moe.moe_pack_weights(w, epilogue) if layout == "packed" else w


def _packed_reference(Wbits, silu):
    """The packed layout of moe_pack_weights (include/moe.h), written out
    element by element from its description: uint16 array of the packed size."""
    E, N, K = Wbits.shape
    NT = -(-(N // 2) // 128) if silu else -(-N // 256)
    KS = -(-K // 32)
    out = np.zeros((E, NT, KS, 256, 32), np.uint16)
    for t in range(NT):
        for r in range(256):
            if silu:
                col = t * 128 + (r % 128)
                if col >= N // 2:
                    continue
                row = col if r < 128 else N // 2 + col
            else:
                row = t * 256 + r
                if row >= N:
                    continue
            for ks in range(KS):
                for c in range(4):
                    k0 = ks * 32 + 8 * c
                    if k0 >= K:
                        continue
                    pos = c ^ ((r >> 2) & 3)
                    out[:, t, ks, r, 8 * pos:8 * pos + 8] = Wbits[:, row, k0:k0 + 8]
    return out.reshape(-1)


@pytest.mark.parametrize("silu,N,K", [(False, 80, 40), (False, 512, 64), (True, 96, 40),
                                      (True, 288, 72)])
def test_pack_layout(moe, dev, silu, N, K):
    """Packed bytes equal the documented layout exactly (ragged N and K
    included: padding is zero)."""
    E = 3
    rng = np.random.default_rng(N + K)
    Wbits = rng.integers(0, 1 << 16, size=(E, N, K), dtype=np.uint16)
    pw = moe.moe_pack_weights(bf16_dev(Wbits, dev), "silu_mul" if silu else "none")
    torch.cuda.synchronize()
    got = pw.data.cpu().numpy().view(np.uint16)
    ref = _packed_reference(Wbits, silu)
    assert got.shape == ref.shape
    assert (got == ref).all()


@pytest.mark.parametrize("N,K", [(80, 48), (272, 208)])
def test_pack_layout_int8(moe, dev, N, K):
    """int8 weights: the same layout in bytes (64 int8 per stage).  Two int8
    columns are viewed as one 16-bit element, which the bf16 reference lays
    out identically."""
    E = 2
    rng = np.random.default_rng(7 * N + K)
    W = rng.integers(-128, 128, size=(E, N, K), dtype=np.int8)
    pw = moe.moe_pack_weights(torch.from_numpy(W).to(dev))
    torch.cuda.synchronize()
    got = pw.data.cpu().numpy().view(np.uint16)
    ref = _packed_reference(W.view(np.uint16), False)
    assert got.shape == ref.shape
    assert (got == ref).all()


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
    cases = [(B, "plain") for B in BLOCKS] + [(B, "packed") for B in BLOCKS if B >= 64]
    for B, layout in cases:
        sb, eb, tot, *_ = _meta(moe, ids, 4, B, dev)
        C = moe.moe_grouped_gemm(
            bf16_dev(synth.f32_to_bf16_bits(x), dev),
            _weights(moe, synth.f32_to_bf16_bits(W), dev, layout, "none"),
            sb, eb, tot, B, 4, a_rows="pair", a_row_div=2, c_dtype=torch.float32)
        torch.cuda.synchronize()
        out = C.cpu().numpy()
        assert out[:, :2].reshape(2, 2, 2).tolist() == g["output"], (B, layout)
        assert (out[:, 2:] == 0).all()


def _rand_case(seed, T, E, K_top, H, N, a_f32=False):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:K_top] for _ in range(T)])
    A = synth.normal_f32((T, H), 9, 0, seed)
    Bw = synth.normal_f32((E, N, H), 9, 1, seed, 0.05)
    wts = rng.random(T * K_top).astype(np.float32)
    return ids, A, Bw, wts


CASES = [(B, "plain") for B in BLOCKS] + [(B, "packed") for B in BLOCKS if B >= 64]


@pytest.mark.parametrize("B,layout", CASES)
@pytest.mark.parametrize("epilogue", ["none", "silu_mul"])
@pytest.mark.parametrize("c_dtype", [torch.float32, torch.bfloat16])
def test_gemm_pair_rows(moe, dev, B, layout, epilogue, c_dtype):
    T, E, Kt, H, N = 97, 7, 3, 136, 96        # K tail (136 = 2 stages + 8), N not /128
    ids, A, Bw, wts = _rand_case(B + (epilogue == "none"), T, E, Kt, H, N)
    Ab, Bb = synth.f32_to_bf16_bits(A), synth.f32_to_bf16_bits(Bw)
    sb, eb, tot, s, e, total = _meta(moe, ids, E, B, dev)
    P = ids.size
    w_dev = torch.from_numpy(wts).to(dev)
    C = torch.full((P, N // 2 if epilogue == "silu_mul" else N), float("nan"),
                   dtype=c_dtype, device=dev)
    moe.moe_grouped_gemm(bf16_dev(Ab, dev), _weights(moe, Bb, dev, layout, epilogue), sb, eb, tot,
                         B, P, a_rows="pair", a_row_div=Kt, topk_weights=w_dev, epilogue=epilogue,
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


def _selector(E, N, H, scale_of_expert):
    """bf16 weights with one nonzero per output column: B[e, n, (3n + e) % H]
    = scale_of_expert(e).  Every output is then one exact product."""
    Bw = np.zeros((E, N, H), np.float32)
    n = np.arange(N)
    for e in range(E):
        Bw[e, n, (3 * n + e) % H] = scale_of_expert(e)
    return synth.f32_to_bf16_bits(Bw)


@pytest.mark.parametrize("B,layout", CASES)
@pytest.mark.parametrize("c_dtype", [torch.bfloat16, torch.float16])
def test_gemm_output_rounding_exact(moe, dev, B, layout, c_dtype):
    """16-bit outputs are the round-to-nearest-even of the float32 result,
    bit for bit.  With a selector weight each output is a * c_e * w, where a
    (bf16), c_e = 1 + (2e+1)/128 and w = 2^-j make a product that float32
    holds exactly but 16 bits do not, ties included; torch's CPU conversion
    of that exact product is the expected value."""
    T, E, Kt, H, N = 89, 7, 3, 64, 96
    ids, A, _, _ = _rand_case(B + 5, T, E, Kt, H, N)
    Ab = synth.f32_to_bf16_bits(A * 3.0)
    Bb = _selector(E, N, H, lambda e: 1.0 + (2 * e + 1) / 128.0)
    P = ids.size
    wts = np.ldexp(1.0, -(np.arange(P) % 4)).astype(np.float32)
    sb, eb, tot, s, e, total = _meta(moe, ids, E, B, dev)
    C = torch.full((P, N), float("nan"), dtype=c_dtype, device=dev)
    moe.moe_grouped_gemm(bf16_dev(Ab, dev), _weights(moe, Bb, dev, layout, "none"), sb, eb, tot, B,
                         P, a_rows="pair", a_row_div=Kt, topk_weights=torch.from_numpy(wts).to(dev),
                         C=C, c_rows="pair")
    torch.cuda.synchronize()
    A64, B64 = oracle.bf16_bits_to_f64(Ab), oracle.bf16_bits_to_f64(Bb)
    exact = np.einsum("pk,pnk->pn", A64[np.arange(P) // Kt], B64[ids.reshape(-1)]) * wts[:, None]
    assert (exact.astype(np.float32).astype(np.float64) == exact).all()   # float32 holds it
    ref = torch.from_numpy(exact.astype(np.float32)).to(c_dtype)
    got = C.cpu()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    # the case does exercise rounding: many products are not 16-bit values
    assert (ref.double().numpy() != exact).mean() > 0.5


@pytest.mark.parametrize("B", [b for b in BLOCKS if b != 256])
def test_gemm_f32_input_rounding_exact(moe, dev, B):
    """float32 tokens are rounded to bf16 on load, to nearest even: with a
    selector weight of 1 the float32 output is exactly torch's bf16 rounding
    of the token value."""
    T, E, Kt, H, N = 61, 5, 2, 64, 48
    ids, A, _, _ = _rand_case(B + 11, T, E, Kt, H, N)
    A = A * np.float32(1.0 + 2.0 ** -9)         # values off the bf16 grid
    Bb = _selector(E, N, H, lambda e: 1.0)
    sb, eb, tot, s, e, total = _meta(moe, ids, E, B, dev)
    P = ids.size
    C = torch.full((P, N), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_grouped_gemm(torch.from_numpy(A).to(dev), bf16_dev(Bb, dev), sb, eb, tot, B, P,
                         a_rows="pair", a_row_div=Kt, C=C, c_rows="pair")
    torch.cuda.synchronize()
    Ar = torch.from_numpy(A).to(torch.bfloat16).float().numpy()
    ex = ids.reshape(-1)
    cols = (3 * np.arange(N)[None, :] + ex[:, None]) % H
    ref = Ar[(np.arange(P) // Kt)[:, None], cols]
    assert np.array_equal(C.cpu().numpy(), ref)


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


@pytest.mark.parametrize("B,layout", CASES)
def test_gemm_skewed_experts(moe, dev, B, layout):
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
    C = moe.moe_grouped_gemm(bf16_dev(Ab, dev), _weights(moe, Bb, dev, layout, "none"), sb, eb,
                             tot, B, T, c_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_gemm_sorted(oracle.bf16_bits_to_f64(Ab), oracle.bf16_bits_to_f64(Bb),
                                        s, e, B, T, 1)
    assert max_abs_rel(C.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("B,layout", [(64, "plain"), (128, "packed"), (256, "plain")])
def test_gemm_long_and_short_experts(moe, dev, B, layout):
    """One expert spans more token blocks than the kernels' tile-order window
    (it keeps block-major tile order), the others span 1-3 blocks (n-tile-major
    order inside the expert); every output row is written exactly once."""
    E, H, N = 6, 64, 512
    counts = [40000, 1, 130, 0, 257, 64]
    ids = np.concatenate([np.full(c, e, np.int64) for e, c in enumerate(counts)])
    ids = np.random.default_rng(B).permutation(ids)[:, None]
    T = ids.shape[0]
    A = synth.normal_f32((T, H), 9, 11)
    Bw = synth.normal_f32((E, N, H), 9, 12, 0, 0.05)
    Ab, Bb = synth.f32_to_bf16_bits(A), synth.f32_to_bf16_bits(Bw)
    sb, eb, tot, s, e, total = _meta(moe, ids, E, B, dev)
    C = torch.full((T, N), float("nan"), dtype=torch.float32, device=dev)
    moe.moe_grouped_gemm(bf16_dev(Ab, dev), _weights(moe, Bb, dev, layout, "none"), sb, eb, tot, B,
                         T, C=C)
    torch.cuda.synchronize()
    ref, _ = oracle.grouped_gemm_sorted(oracle.bf16_bits_to_f64(Ab), oracle.bf16_bits_to_f64(Bb),
                                        s, e, B, T, 1)
    got = C.cpu().numpy()
    assert np.isfinite(got).all()
    assert max_abs_rel(got, ref) <= 1e-5


def test_gemm_packed_rejects_f32_input_and_small_blocks(moe, dev):
    ids = np.zeros((8, 1), np.int64)
    A = torch.zeros((8, 64), dtype=torch.float32, device=dev)
    pw = moe.moe_pack_weights(torch.zeros((1, 32, 64), dtype=torch.bfloat16, device=dev))
    sb, eb, tot, *_ = _meta(moe, ids, 1, 64, dev)
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_gemm(A, pw, sb, eb, tot, 64, 8)
    sb, eb, tot, *_ = _meta(moe, ids, 1, 32, dev)
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_gemm(A.to(torch.bfloat16), pw, sb, eb, tot, 32, 8)
    with pytest.raises(ValueError):                       # packed for another epilogue
        moe.moe_grouped_gemm(A.to(torch.bfloat16), pw, sb, eb, tot, 64, 8, epilogue="silu_mul")


def test_gemm_f32_input_rejected_at_256(moe, dev):
    ids = np.zeros((8, 1), np.int64)
    sb, eb, tot, *_ = _meta(moe, ids, 1, 256, dev)
    A = torch.zeros((8, 64), dtype=torch.float32, device=dev)
    Bw = torch.zeros((1, 32, 64), dtype=torch.bfloat16, device=dev)
    with pytest.raises(moe.MoeError):
        moe.moe_grouped_gemm(A, Bw, sb, eb, tot, 256, 8)

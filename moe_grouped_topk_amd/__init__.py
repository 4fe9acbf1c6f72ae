"""Python binding of libmoe.so, the gfx950 fused-MoE library (include/moe.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Tensors are torch tensors on the current ROCm device; outputs that
are not passed in are allocated with torch.empty (device memory plumbing).
Every call enqueues on torch's current stream and does not synchronise.

The package fails loudly at import if the library has not been built; there
is no CPU fallback.
"""

import ctypes
import os

__all__ = [
    "MoeError", "LIB_PATH", "lib", "moe_status_string", "moe_route",
    "moe_align_max_padded", "moe_align_workspace_size", "moe_align_block_size", "moe_grouped_gemm",
    "moe_forward_block_m", "moe_forward_workspace_size", "moe_forward", "gmm_int8", "DTYPE", "SCORING",
    "EPILOGUE", "ROWS", "WEIGHTS", "moe_packed_weights_size", "moe_pack_weights",
    "PackedWeights", "moe_quantize_rows", "moe_forward_w8a8_workspace_size", "moe_forward_w8a8",
    "moe_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "moe_wide_tile_table_size",
    "moe_wide_tile_table", "moe_grouped_gemm_wide",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

# Codes of include/moe.h
DTYPE = {"f32": 0, "bf16": 1, "f16": 2, "i8": 3}
SCORING = {"softmax": 0, "sigmoid": 1}
EPILOGUE = {"none": 0, "silu_mul": 1}
ROWS = {"pair": 0, "sorted": 1}
WEIGHTS = {"plain": 0, "packed": 1}


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %d (%s)" % (fn, status, moe_status_string(status)))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libmoe.so is not built (%s); build it with "
            "`python moe_grouped_topk_amd/build.py` or __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                             ctypes.c_float, ctypes.c_size_t)
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_route.argtypes = [vp, i64, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp]
    L.moe_route.restype = ctypes.c_int
    L.moe_align_max_padded.argtypes = [i64, i32, i32]
    L.moe_align_max_padded.restype = i64
    L.moe_align_workspace_size.argtypes = [i64, i32]
    L.moe_align_workspace_size.restype = sz
    L.moe_align_block_size.argtypes = [vp, i64, i32, i32, vp, vp, vp, i64, vp, sz, vp]
    L.moe_align_block_size.restype = ctypes.c_int
    L.moe_packed_weights_size.argtypes = [i32, i32, i64, i64, i32]
    L.moe_packed_weights_size.restype = sz
    L.moe_pack_weights.argtypes = [vp, i32, i32, i64, i64, i32, vp, sz, vp]
    L.moe_pack_weights.restype = ctypes.c_int
    L.moe_grouped_gemm.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, i64, i64, vp, vp, vp, i64,
                                   i32, i64, vp, i32, vp, i32, i64, i32, vp]
    L.moe_grouped_gemm.restype = ctypes.c_int
    L.moe_wide_tile_table_size.argtypes = [i64]
    L.moe_wide_tile_table_size.restype = i64
    L.moe_wide_tile_table.argtypes = [vp, vp, i32, i64, vp, i64, vp]
    L.moe_wide_tile_table.restype = ctypes.c_int
    L.moe_grouped_gemm_wide.argtypes = [vp, i32, i64, i32, i32, vp, i32, i32, i64, i64, vp, vp,
                                        vp, i64, vp, i64, vp, i32, vp, i32, i64, i32, vp]
    L.moe_grouped_gemm_wide.restype = ctypes.c_int
    L.moe_forward_block_m.argtypes = [i64, i32, i32, i32, i32]
    L.moe_forward_block_m.restype = i32
    L.moe_forward_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    L.moe_forward_workspace_size.restype = sz
    L.moe_forward.argtypes = [vp, i32, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, i32, i32,
                              i32, f32, i32, vp, vp, vp, vp, sz, vp]
    L.moe_forward.restype = ctypes.c_int
    L.moe_forward_noalloc.argtypes = [vp, i32, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32, i32,
                                      i32, i32, f32, i32, vp, vp, vp, vp]
    L.moe_forward_noalloc.restype = ctypes.c_int
    L.gmm_int8.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    L.moe_quantize_rows.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp]
    L.moe_quantize_rows.restype = ctypes.c_int
    L.moe_forward_w8a8_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    L.moe_forward_w8a8_workspace_size.restype = sz
    L.moe_forward_w8a8.argtypes = [vp, i32, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i32,
                                   i32, i32, i32, f32, i32, vp, vp, vp, vp, sz, vp]
    L.moe_forward_w8a8.restype = ctypes.c_int
    L.gmm_int8.restype = ctypes.c_int
    return L


lib = _load()


def moe_status_string(status):
    return lib.moe_status_string(int(status)).decode()


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status)


def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous torch tensor on the GPU (or None)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dtype_code(t):
    torch = _torch()
    return {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[t.dtype]


def moe_route(gating, topk, num_expert_group=1, topk_group=1, scoring="softmax",
              renormalize=True, routed_scaling_factor=1.0, topk_weights=None,
              topk_ids=None, stream=None):
    """Grouped / plain top-k routing of gating [T, E] float32 logits.
    Returns (topk_weights [T, topk] float32, topk_ids [T, topk] int32)."""
    torch = _torch()
    T, E = gating.shape
    if topk_weights is None:
        topk_weights = torch.empty((T, topk), dtype=torch.float32, device=gating.device)
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=gating.device)
    _check("moe_route", lib.moe_route(
        _ptr(gating, torch.float32, "gating"), T, E, topk, num_expert_group, topk_group,
        SCORING[scoring], int(bool(renormalize)), float(routed_scaling_factor),
        _ptr(topk_weights, torch.float32, "topk_weights"),
        _ptr(topk_ids, torch.int32, "topk_ids"), _stream(stream)))
    return topk_weights, topk_ids


def moe_align_max_padded(num_pairs, num_experts, block_m):
    return int(lib.moe_align_max_padded(int(num_pairs), int(num_experts), int(block_m)))


def moe_align_workspace_size(num_pairs, num_experts):
    return int(lib.moe_align_workspace_size(int(num_pairs), int(num_experts)))


def moe_align_block_size(topk_ids, num_experts, block_m, sorted_token_ids=None,
                         expert_ids=None, num_tokens_post_padded=None, workspace=None,
                         stream=None):
    """Returns (sorted_token_ids [max_padded] int32, expert_ids
    [max_padded // block_m] int32, num_tokens_post_padded [1] int32).
    workspace: optional uint8 device tensor of moe_align_workspace_size
    bytes (selects the two-kernel path; same outputs)."""
    torch = _torch()
    P = topk_ids.numel()
    cap = moe_align_max_padded(P, num_experts, block_m)
    dev = topk_ids.device
    if sorted_token_ids is None:
        sorted_token_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    if expert_ids is None:
        expert_ids = torch.empty(cap // block_m, dtype=torch.int32, device=dev)
    if num_tokens_post_padded is None:
        num_tokens_post_padded = torch.empty(1, dtype=torch.int32, device=dev)
    if expert_ids.numel() < sorted_token_ids.numel() // block_m:
        raise ValueError("expert_ids is smaller than sorted_token_ids / block_m")
    _check("moe_align_block_size", lib.moe_align_block_size(
        _ptr(topk_ids, torch.int32, "topk_ids"), P, num_experts, block_m,
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(expert_ids, torch.int32, "expert_ids"),
        _ptr(num_tokens_post_padded, torch.int32, "num_tokens_post_padded"),
        sorted_token_ids.numel(), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _stream(stream)))
    return sorted_token_ids, expert_ids, num_tokens_post_padded


def moe_packed_weights_size(E, N, K, epilogue="none", dtype="bf16"):
    return int(lib.moe_packed_weights_size(DTYPE[dtype], E, N, K, EPILOGUE[epilogue]))


def moe_pack_weights(w, epilogue="none", packed=None, stream=None):
    """Re-layout expert weights w [E, N, K] (bf16, or int8 for gmm_int8) for
    the tile kernels (see moe_pack_weights in include/moe.h).  Returns a
    PackedWeights holding the packed bytes and the logical shape."""
    torch = _torch()
    E, N, K = w.shape
    dtype = {torch.bfloat16: "bf16", torch.int8: "i8"}.get(w.dtype)
    if dtype is None:
        raise TypeError("w must be bfloat16 or int8, got %s" % w.dtype)
    need = moe_packed_weights_size(E, N, K, epilogue, dtype)
    if need == 0:
        raise MoeError("moe_packed_weights_size", -2)
    if packed is None:
        packed = torch.empty(need, dtype=torch.uint8, device=w.device)
    _check("moe_pack_weights", lib.moe_pack_weights(
        _ptr(w, None, "w"), DTYPE[dtype], E, N, K, EPILOGUE[epilogue],
        _ptr(packed, torch.uint8, "packed"), packed.numel(), _stream(stream)))
    return PackedWeights(packed, (E, N, K), epilogue, dtype)


class PackedWeights:
    """Packed expert weights: `data` (uint8 device tensor) plus the logical
    [E, N, K] shape and the epilogue they were packed for."""

    def __init__(self, data, shape, epilogue, dtype="bf16"):
        self.data, self.shape, self.epilogue, self.dtype = data, tuple(shape), epilogue, dtype

    @property
    def device(self):
        return self.data.device


def _weights(B, epilogue, name):
    """(pointer, layout code, (E, N, K)) of plain or packed weights."""
    torch = _torch()
    if isinstance(B, PackedWeights):
        if B.dtype != "bf16":
            raise TypeError("%s holds packed %s weights, bf16 needed" % (name, B.dtype))
        if B.epilogue != epilogue:
            raise ValueError("%s was packed for epilogue %r, used with %r" % (name, B.epilogue, epilogue))
        return _ptr(B.data, torch.uint8, name), WEIGHTS["packed"], B.shape
    return _ptr(B, torch.bfloat16, name), WEIGHTS["plain"], tuple(B.shape)


def moe_grouped_gemm(A, B, sorted_token_ids, expert_ids, num_tokens_post_padded, block_m,
                     num_valid_pairs, a_rows="pair", a_row_div=1, topk_weights=None,
                     epilogue="none", C=None, c_dtype=None, c_rows="pair", c_num_rows=None,
                     stream=None):
    """Sorted grouped GEMM.  A [rows, K] (bf16 or f32), B [E, N, K] bf16 or
    PackedWeights (packed for the same epilogue).  C is allocated as
    [c_num_rows or (num_valid_pairs if c_rows == 'pair' else
    len(sorted_token_ids)), N or N/2] of c_dtype (default A's dtype)."""
    torch = _torch()
    b_ptr, b_layout, (E, N, K) = _weights(B, epilogue, "B")
    nout = N // 2 if epilogue == "silu_mul" else N
    if C is None:
        rows = c_num_rows if c_num_rows is not None else (
            num_valid_pairs if c_rows == "pair" else sorted_token_ids.numel())
        C = torch.empty((rows, nout), dtype=c_dtype or A.dtype, device=A.device)
    if expert_ids.numel() < sorted_token_ids.numel() // block_m:
        raise ValueError("expert_ids is smaller than sorted_token_ids / block_m")
    _check("moe_grouped_gemm", lib.moe_grouped_gemm(
        _ptr(A, None, "A"), _dtype_code(A), A.shape[-1], ROWS[a_rows], a_row_div,
        b_ptr, b_layout, E, N, K,
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(expert_ids, torch.int32, "expert_ids"),
        _ptr(num_tokens_post_padded, torch.int32, "num_tokens_post_padded"),
        sorted_token_ids.numel(), block_m, num_valid_pairs,
        _ptr(topk_weights, torch.float32, "topk_weights"), EPILOGUE[epilogue],
        _ptr(C, None, "C"), _dtype_code(C), C.shape[-1], ROWS[c_rows], _stream(stream)))
    return C


def moe_wide_tile_table_size(max_padded):
    return int(lib.moe_wide_tile_table_size(int(max_padded)))


def moe_wide_tile_table(expert_ids, num_tokens_post_padded, num_experts, max_padded, table=None,
                        stream=None):
    """Tile table of the expert-wide GEMM tiles from a block-32 alignment
    (int32 [moe_wide_tile_table_size(max_padded)])."""
    torch = _torch()
    n = moe_wide_tile_table_size(max_padded)
    if n < 0:
        raise ValueError("max_padded must be a non-negative multiple of 32")
    if table is None:
        table = torch.empty(n, dtype=torch.int32, device=expert_ids.device)
    _check("moe_wide_tile_table", lib.moe_wide_tile_table(
        _ptr(expert_ids, torch.int32, "expert_ids"),
        _ptr(num_tokens_post_padded, torch.int32, "num_tokens_post_padded"), num_experts,
        max_padded, _ptr(table, torch.int32, "table"), table.numel(), _stream(stream)))
    return table


def moe_grouped_gemm_wide(A, B, sorted_token_ids, expert_ids, num_tokens_post_padded, tile_table,
                          num_valid_pairs, a_rows="pair", a_row_div=1, topk_weights=None,
                          epilogue="none", C=None, c_rows="pair", c_num_rows=None, stream=None):
    """moe_grouped_gemm at block_m 32 on expert-wide tiles (bf16 A and C);
    tile_table from moe_wide_tile_table on the same alignment."""
    torch = _torch()
    b_ptr, b_layout, (E, N, K) = _weights(B, epilogue, "B")
    nout = N // 2 if epilogue == "silu_mul" else N
    if C is None:
        rows = c_num_rows if c_num_rows is not None else (
            num_valid_pairs if c_rows == "pair" else sorted_token_ids.numel())
        C = torch.empty((rows, nout), dtype=torch.bfloat16, device=A.device)
    if expert_ids.numel() < sorted_token_ids.numel() // 32:
        raise ValueError("expert_ids is smaller than sorted_token_ids / 32")
    _check("moe_grouped_gemm_wide", lib.moe_grouped_gemm_wide(
        _ptr(A, None, "A"), _dtype_code(A), A.shape[-1], ROWS[a_rows], a_row_div,
        b_ptr, b_layout, E, N, K,
        _ptr(sorted_token_ids, torch.int32, "sorted_token_ids"),
        _ptr(expert_ids, torch.int32, "expert_ids"),
        _ptr(num_tokens_post_padded, torch.int32, "num_tokens_post_padded"),
        sorted_token_ids.numel(), _ptr(tile_table, torch.int32, "tile_table"), num_valid_pairs,
        _ptr(topk_weights, torch.float32, "topk_weights"), EPILOGUE[epilogue],
        _ptr(C, None, "C"), _dtype_code(C), C.shape[-1], ROWS[c_rows], _stream(stream)))
    return C


def moe_forward_block_m(T, E, topk, x_dtype="bf16", weights="plain"):
    """Block size moe_forward picks for block_m=0."""
    return int(lib.moe_forward_block_m(T, E, topk, DTYPE[x_dtype], WEIGHTS[weights]))


def moe_forward_workspace_size(T, H, I, E, topk, block_m=0):
    return int(lib.moe_forward_workspace_size(T, H, I, E, topk, block_m))


def moe_forward(x, gating, w1, w2, topk, num_expert_group=1, topk_group=1,
                scoring="softmax", renormalize=True, routed_scaling_factor=1.0,
                block_m=0, out=None, topk_weights_out=None, topk_ids_out=None,
                workspace=None, stream=None):
    """Whole fused-MoE layer: x [T, H] (bf16 or f32), gating [T, E] f32,
    w1 [E, 2I, H] bf16, w2 [E, H, I] bf16, both plain or both PackedWeights
    (w1 packed for 'silu_mul', w2 for 'none').  Returns out [T, H] in x's dtype."""
    torch = _torch()
    T, H = x.shape
    w1_ptr, l1, (E, twoI, _) = _weights(w1, "silu_mul", "w1")
    w2_ptr, l2, _ = _weights(w2, "none", "w2")
    if l1 != l2:
        raise ValueError("w1 and w2 must both be plain or both packed")
    I = twoI // 2
    if out is None:
        out = torch.empty_like(x)
    need = moe_forward_workspace_size(T, H, I, E, topk, block_m)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check("moe_forward", lib.moe_forward(
        _ptr(x, None, "x"), _dtype_code(x), _ptr(gating, torch.float32, "gating"),
        w1_ptr, w2_ptr, l1, T, H, I, E, topk,
        num_expert_group, topk_group, SCORING[scoring], int(bool(renormalize)),
        float(routed_scaling_factor), block_m, _ptr(out, x.dtype, "out"),
        _ptr(topk_weights_out, torch.float32, "topk_weights_out"),
        _ptr(topk_ids_out, torch.int32, "topk_ids_out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 96 << 20     # MOE_NOALLOC_SCRATCH_BYTES of moe.h


def moe_forward_noalloc(x, gating, w1, w2, topk, out, num_expert_group=1, topk_group=1,
                        scoring="softmax", renormalize=True, routed_scaling_factor=1.0,
                        block_m=0, topk_weights_out=None, topk_ids_out=None, stream=None):
    """moe_forward on the library's static per-device scratch: nothing is
    allocated, here or in the library, so `out` [T, H] (x's dtype) must be
    given.  Calls that overlap on one device race on the scratch."""
    torch = _torch()
    T, H = x.shape
    w1_ptr, l1, (E, twoI, _) = _weights(w1, "silu_mul", "w1")
    w2_ptr, l2, _ = _weights(w2, "none", "w2")
    if l1 != l2:
        raise ValueError("w1 and w2 must both be plain or both packed")
    if out is None:
        raise ValueError("moe_forward_noalloc needs the output tensor")
    _check("moe_forward_noalloc", lib.moe_forward_noalloc(
        _ptr(x, None, "x"), _dtype_code(x), _ptr(gating, torch.float32, "gating"),
        w1_ptr, w2_ptr, l1, T, H, twoI // 2, E, topk,
        num_expert_group, topk_group, SCORING[scoring], int(bool(renormalize)),
        float(routed_scaling_factor), block_m, _ptr(out, x.dtype, "out"),
        _ptr(topk_weights_out, torch.float32, "topk_weights_out"),
        _ptr(topk_ids_out, torch.int32, "topk_ids_out"), _stream(stream)))
    return out


def gmm_int8(input, weights, scales_x, scales_w, expert_offsets, expert_sizes=None,
             output=None, stream=None):
    """INT8 grouped GEMM: input [M, K] int8 sorted by expert, weights [E, N, K]
    int8 (or PackedWeights packed from them), scales_x [M] f32, scales_w [E, N]
    f32, expert_offsets [E+1] int32.  Returns output [M, N] float16."""
    torch = _torch()
    M, K = input.shape
    if isinstance(weights, PackedWeights):
        if weights.dtype != "i8" or weights.epilogue != "none":
            raise TypeError("weights must be int8 weights packed with epilogue 'none'")
        E, N, _ = weights.shape
        w_ptr, w_layout = _ptr(weights.data, torch.uint8, "weights"), WEIGHTS["packed"]
    else:
        E, N, _ = weights.shape
        w_ptr, w_layout = _ptr(weights, torch.int8, "weights"), WEIGHTS["plain"]
    if output is None:
        output = torch.empty((M, N), dtype=torch.float16, device=input.device)
    _check("gmm_int8", lib.gmm_int8(
        _ptr(input, torch.int8, "input"), w_ptr, w_layout,
        _ptr(scales_x, torch.float32, "scales_x"), _ptr(scales_w, torch.float32, "scales_w"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(expert_sizes, torch.int32, "expert_sizes"), _ptr(output, torch.float16, "output"),
        M, K, N, E, _stream(stream)))
    return output


def moe_quantize_rows(x, q=None, scales=None, stream=None):
    """Symmetric per-row int8 quantisation of x [rows, cols] (f32 or bf16;
    rows may be strided).  Returns (q [rows, cols] int8, scales [rows] float32)."""
    torch = _torch()
    rows, cols = x.shape
    if not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a GPU tensor with contiguous rows")
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    _check("moe_quantize_rows", lib.moe_quantize_rows(
        x.data_ptr(), _dtype_code(x), rows, cols, x.stride(0), _ptr(q, torch.int8, "q"),
        _ptr(scales, torch.float32, "scales"), _stream(stream)))
    return q, scales


def moe_forward_w8a8_workspace_size(T, H, I, E, topk, block_m=0):
    return int(lib.moe_forward_w8a8_workspace_size(T, H, I, E, topk, block_m))


def _int8_weights(w, epilogue, name):
    torch = _torch()
    if isinstance(w, PackedWeights):
        if w.dtype != "i8" or w.epilogue != epilogue:
            raise TypeError("%s must be int8 weights packed for epilogue %r" % (name, epilogue))
        return _ptr(w.data, torch.uint8, name), WEIGHTS["packed"], w.shape
    return _ptr(w, torch.int8, name), WEIGHTS["plain"], tuple(w.shape)


def moe_forward_w8a8(x, gating, w1q, w1_scales, w2q, w2_scales, topk, num_expert_group=1,
                     topk_group=1, scoring="softmax", renormalize=True,
                     routed_scaling_factor=1.0, block_m=0, out=None, topk_weights_out=None,
                     topk_ids_out=None, workspace=None, stream=None):
    """Fused-MoE layer with int8 weights (w1q [E, 2I, H], w2q [E, H, I], plain
    int8 tensors or both PackedWeights) and per-channel f32 scales
    (w1_scales [E, 2I], w2_scales [E, H]); activations are quantised per
    token inside.  Returns out [T, H] in x's dtype."""
    torch = _torch()
    T, H = x.shape
    w1_ptr, l1, (E, twoI, _) = _int8_weights(w1q, "silu_mul", "w1q")
    w2_ptr, l2, _ = _int8_weights(w2q, "none", "w2q")
    if l1 != l2:
        raise ValueError("w1q and w2q must both be plain or both packed")
    I = twoI // 2
    if out is None:
        out = torch.empty_like(x)
    need = moe_forward_w8a8_workspace_size(T, H, I, E, topk, block_m)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _check("moe_forward_w8a8", lib.moe_forward_w8a8(
        _ptr(x, None, "x"), _dtype_code(x), _ptr(gating, torch.float32, "gating"),
        w1_ptr, _ptr(w1_scales, torch.float32, "w1_scales"), w2_ptr,
        _ptr(w2_scales, torch.float32, "w2_scales"), l1, T, H, I, E, topk,
        num_expert_group, topk_group, SCORING[scoring], int(bool(renormalize)),
        float(routed_scaling_factor), block_m, _ptr(out, x.dtype, "out"),
        _ptr(topk_weights_out, torch.float32, "topk_weights_out"),
        _ptr(topk_ids_out, torch.int32, "topk_ids_out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))
    return out

"""Host-side checks of the C ABI library that need no GPU: it loads, exports
every entry point include/moe.h declares, and its pure host functions and
argument validation behave as documented (validation returns before any HIP
call is made)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def _defines():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(MOE_\w+)\s+(-?\d+)", text)}


@pytest.fixture(scope="module")
def mod():
    import moe_grouped_topk_amd as m
    return m


def test_header_declares_five_path_calls():
    names = _declared()
    for n in ["moe_route", "moe_align_block_size", "moe_grouped_gemm", "moe_forward",
              "gmm_int8"]:
        assert n in names


def test_library_exports_every_declared_symbol(mod):
    lib = ctypes.CDLL(mod.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_only_declared_symbols_exported(mod):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", mod.LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(_declared())


def test_codes_match_binding(mod):
    d = _defines()
    assert d["MOE_DTYPE_F32"] == mod.DTYPE["f32"] and d["MOE_DTYPE_BF16"] == mod.DTYPE["bf16"]
    assert d["MOE_DTYPE_F16"] == mod.DTYPE["f16"] and d["MOE_DTYPE_I8"] == mod.DTYPE["i8"]
    assert d["MOE_SCORING_SOFTMAX"] == mod.SCORING["softmax"]
    assert d["MOE_SCORING_SIGMOID"] == mod.SCORING["sigmoid"]


def test_status_strings(mod):
    d = _defines()
    assert mod.moe_status_string(0) == "ok"
    seen = set()
    for k, v in d.items():
        if k.startswith("MOE_ERR_"):
            s = mod.moe_status_string(v)
            assert s and s != "unknown status"
            seen.add(s)
    assert len(seen) == 6
    assert mod.moe_status_string(12345) == "unknown status"


def test_align_max_padded_bound(mod):
    import oracle
    import numpy as np
    for P, E, B in [(0, 4, 16), (10, 8, 4), (128, 256, 16), (32768, 128, 128), (5, 1, 1)]:
        got = mod.moe_align_max_padded(P, E, B)
        assert got == oracle.align_max_padded(P, E, B)
        assert got % B == 0
    # the bound holds for adversarial counts (every expert count = 1 mod B)
    rng = np.random.default_rng(0)
    for _ in range(50):
        E = int(rng.integers(1, 30)); B = int(rng.integers(1, 20))
        ids = rng.integers(0, E, size=int(rng.integers(0, 60)))
        _, _, total = oracle.moe_align_block_size(ids, E, B)
        assert total <= mod.moe_align_max_padded(ids.size, E, B)
    assert mod.moe_align_max_padded(-1, 4, 4) == -1


def test_workspace_size(mod):
    ws = mod.moe_forward_workspace_size(4096, 2048, 768, 128, 8)
    P = 4096 * 8
    maxp = mod.moe_align_max_padded(P, 128, 128)
    assert ws >= 4 * P * 2 + 4 * maxp + 2 * maxp * 768 + 4 * P * 2048
    assert ws % 256 == 0
    assert mod.lib.moe_forward_workspace_size(16, 7168, 2048, 256, 8, 48) == 0   # bad block_m
    # covers the packed-weight choice of block size (at least 64) too
    P = 16 * 8
    assert mod.moe_forward_workspace_size(16, 7168, 2048, 256, 8) >= \
        2 * mod.moe_align_max_padded(P, 256, 64) * 2048


# ---- validation error paths (no HIP call is reached) -----------------------

def test_route_validation(mod):
    L, d = mod.lib, _defines()
    fake = ctypes.c_void_p(256)
    # E % G != 0
    assert L.moe_route(fake, 4, 30, 2, 4, 2, 0, 1, 1.0, fake, fake, None) == d["MOE_ERR_CONFIG"]
    # topk > Kg * E/G
    assert L.moe_route(fake, 4, 32, 9, 4, 1, 0, 1, 1.0, fake, fake, None) == d["MOE_ERR_CONFIG"]
    # topk_group > G
    assert L.moe_route(fake, 4, 32, 2, 4, 5, 0, 1, 1.0, fake, fake, None) == d["MOE_ERR_CONFIG"]
    # bad scoring
    assert L.moe_route(fake, 4, 32, 2, 1, 1, 7, 1, 1.0, fake, fake, None) == d["MOE_ERR_CONFIG"]
    # E too large, topk too large
    assert L.moe_route(fake, 4, 2048, 2, 1, 1, 0, 1, 1.0, fake, fake, None) == d["MOE_ERR_SHAPE"]
    assert L.moe_route(fake, 4, 256, 65, 1, 1, 0, 1, 1.0, fake, fake, None) == d["MOE_ERR_SHAPE"]
    # null outputs
    assert L.moe_route(fake, 4, 32, 2, 1, 1, 0, 1, 1.0, None, fake, None) == d["MOE_ERR_NULL"]
    assert L.moe_route(None, 4, 32, 2, 1, 1, 0, 1, 1.0, fake, fake, None) == d["MOE_ERR_NULL"]
    assert L.moe_route(fake, -1, 32, 2, 1, 1, 0, 1, 1.0, fake, fake, None) == d["MOE_ERR_SHAPE"]


def test_align_validation(mod):
    L, d = mod.lib, _defines()
    f = ctypes.c_void_p(256)
    assert L.moe_align_block_size(f, 10, 8, 4, None, f, f, 36, None, 0, None) == d["MOE_ERR_NULL"]
    assert L.moe_align_block_size(None, 10, 8, 4, f, f, f, 36, None, 0, None) == d["MOE_ERR_NULL"]
    assert L.moe_align_block_size(f, 10, 8, 4, f, f, f, 35, None, 0, None) == d["MOE_ERR_SHAPE"]
    assert L.moe_align_block_size(f, 10, 2000, 4, f, f, f, 1 << 20, None, 0,
                                  None) == d["MOE_ERR_SHAPE"]
    assert L.moe_align_block_size(f, 10, 8, 0, f, f, f, 36, None, 0, None) == d["MOE_ERR_CONFIG"]
    need = mod.moe_align_workspace_size(10, 8)
    assert need >= 8 * 4
    assert L.moe_align_block_size(f, 10, 8, 4, f, f, f, 36, f, need - 4,
                                  None) == d["MOE_ERR_WORKSPACE"]
    assert mod.moe_align_workspace_size(-1, 8) == 0


def test_gemm_validation(mod):
    L, d = mod.lib, _defines()
    f = ctypes.c_void_p(256)
    base = dict(A=f, a_dtype=1, lda=128, a_rows=0, a_row_div=2, B=f, bl=0, E=8, N=256, K=128,
                s=f, e=f, tot=f, maxp=512, bm=64, nv=128, w=None, epi=1, C=f, c_dtype=1,
                ldc=128, c_rows=1)

    def call(**kw):
        a = dict(base, **kw)
        return L.moe_grouped_gemm(a["A"], a["a_dtype"], a["lda"], a["a_rows"], a["a_row_div"],
                                  a["B"], a["bl"], a["E"], a["N"], a["K"], a["s"], a["e"],
                                  a["tot"], a["maxp"], a["bm"], a["nv"], a["w"], a["epi"],
                                  a["C"], a["c_dtype"], a["ldc"], a["c_rows"], None)
    assert call(A=None) == d["MOE_ERR_NULL"]
    assert call(a_dtype=2) == d["MOE_ERR_DTYPE"]
    assert call(c_dtype=9) == d["MOE_ERR_DTYPE"]
    assert call(bm=48) == d["MOE_ERR_CONFIG"]
    assert call(epi=5) == d["MOE_ERR_CONFIG"]
    assert call(a_row_div=0) == d["MOE_ERR_CONFIG"]
    assert call(K=100) == d["MOE_ERR_SHAPE"]
    assert call(N=48) == d["MOE_ERR_SHAPE"]            # silu: N/2 % 16
    assert call(lda=64) == d["MOE_ERR_SHAPE"]
    assert call(ldc=64) == d["MOE_ERR_SHAPE"]
    assert call(A=ctypes.c_void_p(264)) == d["MOE_ERR_SHAPE"]   # misaligned
    assert call(bl=2) == d["MOE_ERR_CONFIG"]                     # unknown weight layout
    assert call(bl=1, bm=32) == d["MOE_ERR_CONFIG"]              # packed needs a tile kernel
    assert call(bl=1, a_dtype=0) == d["MOE_ERR_CONFIG"]          # packed needs bf16 A


def test_forward_validation(mod):
    L, d = mod.lib, _defines()
    f = ctypes.c_void_p(256)
    args = [f, 1, f, f, f, 0, 64, 128, 256, 8, 2, 1, 1, 0, 1, 1.0, 0, f, None, None, f, 1 << 30,
            None]
    assert L.moe_forward(*args[:1], 5, *args[2:]) == d["MOE_ERR_DTYPE"]
    a = list(args); a[20] = None
    assert L.moe_forward(*a) == d["MOE_ERR_WORKSPACE"]
    a = list(args); a[21] = 1024
    assert L.moe_forward(*a) == d["MOE_ERR_WORKSPACE"]
    a = list(args); a[7] = 100      # H % 16
    assert L.moe_forward(*a) == d["MOE_ERR_SHAPE"]
    a = list(args); a[16] = 24      # block_m
    assert L.moe_forward(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[0] = None
    assert L.moe_forward(*a) == d["MOE_ERR_NULL"]
    a = list(args); a[5] = 3        # weight layout
    assert L.moe_forward(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[5] = 1; a[1] = 0      # packed weights with f32 x
    assert L.moe_forward(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[5] = 1; a[16] = 16    # packed weights with the streaming block size
    assert L.moe_forward(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[5] = 1; a[1] = 0; a[16] = 32   # block 32 packed: bf16 x only (wide tiles)
    assert L.moe_forward(*a) == d["MOE_ERR_CONFIG"]


def test_forward_noalloc_validation(mod):
    """The allocation-free layer call validates like moe_forward, and rejects
    a layer whose workspace exceeds the static scratch before touching HIP."""
    L, d = mod.lib, _defines()
    text = open(HEADER).read()
    m = re.search(r"#define\s+MOE_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mod.NOALLOC_SCRATCH_BYTES
    f = ctypes.c_void_p(256)
    args = [f, 1, f, f, f, 0, 64, 128, 256, 8, 2, 1, 1, 0, 1, 1.0, 0, f, None, None, None]
    assert L.moe_forward_noalloc(*args[:1], 5, *args[2:]) == d["MOE_ERR_DTYPE"]
    a = list(args); a[7] = 100      # H % 16
    assert L.moe_forward_noalloc(*a) == d["MOE_ERR_SHAPE"]
    a = list(args); a[16] = 24      # block_m
    assert L.moe_forward_noalloc(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[0] = None
    assert L.moe_forward_noalloc(*a) == d["MOE_ERR_NULL"]
    a = list(args); a[6] = 0        # no tokens: nothing to do
    assert L.moe_forward_noalloc(*a) == d["MOE_OK"]
    # the prefill layer needs about 328 MiB of workspace: more than the scratch
    big = [4096, 2048, 768, 128, 8]
    assert mod.moe_forward_workspace_size(*big) > mod.NOALLOC_SCRATCH_BYTES
    a = list(args); a[6:11] = big
    assert L.moe_forward_noalloc(*a) == d["MOE_ERR_WORKSPACE"]
    # decode at T = 64 (H = 7168, I = 2048, E = 256, top-8) fits
    assert mod.moe_forward_workspace_size(64, 7168, 2048, 256, 8) <= mod.NOALLOC_SCRATCH_BYTES


def test_packed_weights_size_and_validation(mod):
    L, d = mod.lib, _defines()
    f = ctypes.c_void_p(256)
    # gate_up of the prefill layer: 6 tiles of 128 gate + 128 up rows, 64 K stages
    assert mod.moe_packed_weights_size(128, 1536, 2048, "silu_mul") == 128 * 6 * 64 * 16384
    assert mod.moe_packed_weights_size(128, 2048, 768, "none") == 128 * 8 * 24 * 16384
    # ragged: N and K rounded up to whole tiles and stages (zero padded)
    assert mod.moe_packed_weights_size(3, 80, 40, "none") == 3 * 1 * 2 * 16384
    assert mod.moe_packed_weights_size(3, 96, 40, "silu_mul") == 3 * 1 * 2 * 16384
    # int8 GMM weights: 64 int8 per stage
    assert mod.moe_packed_weights_size(32, 4096, 4096, "none", "i8") == 32 * 16 * 64 * 16384
    assert mod.moe_packed_weights_size(2, 272, 80, "none", "i8") == 2 * 2 * 2 * 16384
    assert L.moe_packed_weights_size(3, 2, 64, 64, 1) == 2 * 1 * 1 * 16384   # int8 gate/up pairs
    assert L.moe_packed_weights_size(3, 2, 64, 40, 0) == 0               # int8: K % 16
    assert L.moe_packed_weights_size(1, 3, 80, 44, 0) == 0               # K % 8
    assert L.moe_packed_weights_size(1, 3, 48, 40, 1) == 0               # silu: (N/2) % 16
    assert L.moe_packed_weights_size(0, 3, 80, 40, 0) == 0               # f32 weights
    assert L.moe_pack_weights(f, 1, 3, 80, 40, 0, None, 1 << 20, None) == d["MOE_ERR_NULL"]
    assert L.moe_pack_weights(f, 1, 3, 80, 40, 0, f, 16384, None) == d["MOE_ERR_SHAPE"]
    assert L.moe_pack_weights(f, 1, 3, 80, 40, 7, f, 1 << 20, None) == d["MOE_ERR_CONFIG"]
    assert L.moe_pack_weights(f, 2, 3, 80, 40, 0, f, 1 << 20, None) == d["MOE_ERR_DTYPE"]
    assert L.moe_pack_weights(f, 3, 3, 80, 64, 1, f, 1 << 20, None) == d["MOE_ERR_SHAPE"]  # N % 32
    assert L.moe_pack_weights(ctypes.c_void_p(264), 1, 3, 80, 40, 0, f, 1 << 20,
                              None) == d["MOE_ERR_SHAPE"]


def test_quantize_rows_validation(mod):
    L, d = mod.lib, _defines()
    f = ctypes.c_void_p(256)
    assert L.moe_quantize_rows(f, 3, 4, 64, 64, f, f, None) == d["MOE_ERR_DTYPE"]
    assert L.moe_quantize_rows(f, 1, 4, 60, 64, f, f, None) == d["MOE_ERR_SHAPE"]    # cols % 8
    assert L.moe_quantize_rows(f, 1, 4, 64, 32, f, f, None) == d["MOE_ERR_SHAPE"]    # ld < cols
    assert L.moe_quantize_rows(f, 1, 4, 64, 68, f, f, None) == d["MOE_ERR_SHAPE"]    # ld % 8
    assert L.moe_quantize_rows(None, 1, 4, 64, 64, f, f, None) == d["MOE_ERR_NULL"]
    assert L.moe_quantize_rows(ctypes.c_void_p(264), 1, 4, 64, 64, f, f, None) == d["MOE_ERR_SHAPE"]
    assert L.moe_quantize_rows(None, 1, 0, 64, 64, None, None, None) == 0          # no rows


def test_forward_w8a8_validation(mod):
    L, d = mod.lib, _defines()
    f = ctypes.c_void_p(256)
    ws = mod.moe_forward_w8a8_workspace_size(64, 128, 256, 8, 2)
    assert ws > 0 and ws % 256 == 0
    assert mod.lib.moe_forward_w8a8_workspace_size(64, 128, 256, 8, 2, 16) == 0   # block_m < 32
    assert mod.lib.moe_forward_w8a8_workspace_size(64, 128, 256, 8, 2, 32) > 0    # wide int8 tiles
    args = [f, 1, f, f, f, f, f, 0, 64, 128, 256, 8, 2, 1, 1, 0, 1, 1.0, 0, f, None, None, f,
            1 << 30, None]
    a = list(args); a[1] = 2
    assert L.moe_forward_w8a8(*a) == d["MOE_ERR_DTYPE"]
    a = list(args); a[7] = 5
    assert L.moe_forward_w8a8(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[18] = 16
    assert L.moe_forward_w8a8(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[18] = 32; a[1] = 0   # block 32 (the wide int8 tiles) needs bf16 x
    assert L.moe_forward_w8a8(*a) == d["MOE_ERR_CONFIG"]
    a = list(args); a[9] = 120      # H % 16
    assert L.moe_forward_w8a8(*a) == d["MOE_ERR_SHAPE"]
    a = list(args); a[4] = None     # w1_scales
    assert L.moe_forward_w8a8(*a) == d["MOE_ERR_NULL"]
    a = list(args); a[22] = None
    assert L.moe_forward_w8a8(*a) == d["MOE_ERR_WORKSPACE"]
    a = list(args); a[8] = 0        # T = 0
    assert L.moe_forward_w8a8(*a) == 0


def test_gmm_validation(mod):
    L, d = mod.lib, _defines()
    f = ctypes.c_void_p(256)
    assert L.gmm_int8(f, f, 0, f, f, f, None, f, 2048, 4008, 4096, 32, None) == d["MOE_ERR_SHAPE"]
    assert L.gmm_int8(f, f, 0, f, f, f, None, f, 2048, 4096, 4100, 32, None) == d["MOE_ERR_SHAPE"]
    assert L.gmm_int8(f, f, 0, f, f, f, None, f, 2048, 4096, 4096, 0, None) == d["MOE_ERR_SHAPE"]
    assert L.gmm_int8(f, None, 0, f, f, f, None, f, 2048, 4096, 4096, 32, None) == d["MOE_ERR_NULL"]
    assert L.gmm_int8(f, f, 0, f, f, f, None, f, 2048, 1 << 20, 4096, 32, None) == d["MOE_ERR_SHAPE"]
    assert L.gmm_int8(f, f, 2, f, f, f, None, f, 2048, 4096, 4096, 32, None) == d["MOE_ERR_CONFIG"]
    assert L.gmm_int8(None, f, 0, None, f, f, None, None, 0, 4096, 4096, 32, None) == 0   # M = 0


def test_forward_block_m_choice(mod):
    assert mod.moe_forward_block_m(4096, 128, 8) == 32           # prefill shape: expert-wide tiles
    assert mod.moe_forward_block_m(4096, 128, 8, "f32") == 128   # f32 x: 256 x 128 tiles
    assert mod.moe_forward_block_m(1536, 128, 8) == 32           # 96 pairs per expert
    assert mod.moe_forward_block_m(1535, 128, 8) == 64
    assert mod.moe_forward_block_m(32768, 2048, 8) == 128        # more experts than the table takes
    assert mod.moe_forward_block_m(16, 256, 8) == 64             # decode shape, bf16 x
    assert mod.moe_forward_block_m(16, 256, 8, "f32") == 16      # f32 x, plain weights
    assert mod.moe_forward_block_m(64, 8, 2, "f32") == 32        # tiny layer
    assert mod.moe_forward_block_m(16, 256, 8, weights="packed") == 64    # tile kernels only
    assert mod.moe_forward_block_m(4096, 128, 8, weights="packed") == 32
    assert mod.lib.moe_forward_block_m(16, 0, 8, 1, 0) == -1
    assert mod.lib.moe_forward_block_m(16, 256, 8, 1, 5) == -1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message before
    touching torch or the GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_wide_gemm_validation(mod):
    """Argument checks of the expert-wide tile entry points (no GPU work)."""
    L, d = mod.lib, _defines()
    assert L.moe_wide_tile_table_size(320) == 31
    assert L.moe_wide_tile_table_size(0) == 1
    assert L.moe_wide_tile_table_size(33) == -1
    assert L.moe_wide_tile_table_size(-32) == -1
    f = ctypes.c_void_p(256)
    assert L.moe_wide_tile_table(f, f, 0, 320, f, 31, None) == d["MOE_ERR_CONFIG"]
    assert L.moe_wide_tile_table(f, f, 1025, 320, f, 31, None) == d["MOE_ERR_CONFIG"]
    assert L.moe_wide_tile_table(f, f, 8, 320, f, 30, None) == d["MOE_ERR_WORKSPACE"]
    assert L.moe_wide_tile_table(f, f, 8, 330, f, 31, None) == d["MOE_ERR_SHAPE"]
    assert L.moe_wide_tile_table(f, None, 8, 320, f, 31, None) == d["MOE_ERR_NULL"]
    assert L.moe_wide_tile_table(f, f, 8, 320, None, 31, None) == d["MOE_ERR_NULL"]
    # A, a_dtype, lda, a_rows, a_row_div, B, b_layout, E, N, K, sorted, eids, total,
    # max_padded, table, num_valid, topk_weights, epilogue, C, c_dtype, ldc, c_rows, stream
    base = [f, 1, 128, 0, 2, f, 0, 8, 256, 128, f, f, f, 320, f, 100, None, 1, f, 1, 128, 1,
            None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[{"a_dtype": 1, "E": 7, "table": 14, "w": 16, "epi": 17, "c_dtype": 19,
               "bl": 6, "K": 9}[k]] = v
        return L.moe_grouped_gemm_wide(*a)
    assert call(a_dtype=0) == d["MOE_ERR_DTYPE"]                # f32 A
    assert call(c_dtype=0) == d["MOE_ERR_DTYPE"]                # f32 C
    assert call(w=f) == d["MOE_ERR_CONFIG"]                     # SiLU takes no weights
    assert call(E=1025) == d["MOE_ERR_CONFIG"]
    assert call(bl=2) == d["MOE_ERR_CONFIG"]
    assert call(K=100) == d["MOE_ERR_SHAPE"]
    assert call(table=None) == d["MOE_ERR_NULL"]


def test_build_rejects_scratch_use():
    """build.py fails on any kernel whose resource report shows VGPR spills or
    scratch memory (the GEMM loops' load counts assume no scratch traffic);
    SGPR spills, which stay in VGPR lanes, pass."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "moe_build", os.path.join(ROOT, "moe_grouped_topk_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    tag = " [-Rpass-analysis=kernel-resource-usage]"
    log = "\n".join("k.hip:1:2: remark: " + l + tag for l in [
        "Function Name: kA", "    ScratchSize [bytes/lane]: 0", "    SGPRs Spill: 30",
        "    VGPRs Spill: 0",
        "Function Name: kB", "    ScratchSize [bytes/lane]: 32", "    VGPRs Spill: 7"])
    bad = b.check_scratch([log])
    assert bad == ["kB: ScratchSize [bytes/lane] 32", "kB: VGPRs Spill 7"]
    assert b.check_scratch([log.split("Function Name: kB")[0]]) == []

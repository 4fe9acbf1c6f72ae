"""Plain, slow CPU oracle of the fused-MoE forward path (test infrastructure).

This package is TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The HIP library and
its Python binding never import, call or link anything here, and nothing here
imports the HIP path.  Arithmetic is NumPy float64 unless a page fixes another
precision (the int8 GMM accumulates exactly in int64).

Sources, cited in every docstring by these tags (section names as on the page):

[P1]  DatenLord, "From loops to fusion: the Fused MoE operator, Part 3"
      (community.aijishu.com/a/1060000000523566): §01 (the gathered-weight
      bottleneck), §03.1-§03.3 (the index-fused kernel and its worked example).
[GTK] "GroupedTopK operator optimisation primer: from MoE routing to a fused
      Triton kernel" (blog.freezetheflame.cc, 2026-07-27): §二 interface,
      §三 3.1-3.6 step-by-step semantics, §四 hand-worked example, §七 math
      shortcut, §八 Top-K pitfalls, §九 test matrix and invariants.
[MSG] mini-sglang handbook, "MoE and fused MoE"
      (anrans.github.io/ai-infra-handbooks/minisgl/perf/moe/): "路由"
      (select_experts), "参考后端" (TorchMoeBackend), "fused MoE"
      (moe_align_block_size, fused_moe_kernel, FusedMoeBackend.forward),
      "在 CPU 上运行 Triton" (seeded example printout), "练习" and answers.
[GMM] Low-precision grouped GEMM article (www.pwwt.cn/news/5863887/):
      §2.1 definition, §2.2 arithmetic intensity, §2.3 error sources,
      §3.1 interface, §3.2 quantisation, §4 in-kernel quantisation,
      §5.3 INT8 accumulation.

Functions whose result has a plain definition are that definition written out;
none of them is blocked, fused or reordered beyond what the passage states.
"""

from .routing import (softmax_scores, sigmoid_scores, grouped_topk,
                      select_experts)
from .align import moe_align_block_size, align_max_padded
from .gemm import grouped_gemm_sorted, index_fused_gemm, silu, silu_and_mul
from .layer import (moe_layer_expert_loop, moe_layer_pair_rows, moe_layer_token_loop,
                    moe_forward, dense_swiglu)
from .gmm import gmm, gmm_int8, quantize_weight_per_channel, quantize_per_token
from .quant_layer import (quantize_rows_f32, moe_layer_w8a8_expert_loop,
                          moe_layer_w8a8_token_loop)
from .bf16 import bf16_bits_to_f64

__all__ = [
    "softmax_scores", "sigmoid_scores", "grouped_topk", "select_experts",
    "moe_align_block_size", "align_max_padded",
    "grouped_gemm_sorted", "index_fused_gemm", "silu", "silu_and_mul",
    "moe_layer_expert_loop", "moe_layer_pair_rows", "moe_layer_token_loop", "moe_forward",
    "dense_swiglu", "gmm", "gmm_int8", "quantize_weight_per_channel",
    "quantize_per_token", "bf16_bits_to_f64", "quantize_rows_f32",
    "moe_layer_w8a8_expert_loop", "moe_layer_w8a8_token_loop",
]

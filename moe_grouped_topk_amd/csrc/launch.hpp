// Internal kernel launchers (host side).  Each returns hipGetLastError()
// after enqueueing; arguments are validated by the C ABI layer beforehand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Optional work of the routing launch for the int8 layer: each token's row
// of x quantised per row as it is loaded (x_dtype 1 bf16, 0 f32; cols % 8
// == 0, rows 16-byte aligned) into q / scales, and nzero ints at zero set to
// 0 (counters of a later launch).
struct RouteExtra {
  const void* x;
  int x_dtype;
  int64_t cols;
  int8_t* q;
  float* scales;
  int32_t* zero;
  int64_t nzero;
};

// Raises `kernel`'s dynamic-LDS limit on the current device to `bytes` when
// a launch needs more than 64 KiB and more than was raised there before
// (hipFuncSetAttribute once per kernel, device and larger size; the sizes
// already raised are kept in a table for the life of the process).
hipError_t raise_lds_limit(const void* kernel, size_t bytes);

hipError_t launch_route(const float* gating, int64_t T, int E, int topk, int G,
                        int topk_group, int scoring, int renormalize, float scale,
                        float* out_w, int32_t* out_ids, hipStream_t stream,
                        const RouteExtra* extra = nullptr);

hipError_t launch_align(const int32_t* topk_ids, int64_t P, int E, int B,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* total,
                        int64_t max_padded, hipStream_t stream);

// The same alignment in two kernels (per-chunk counts, then placement),
// with a workspace of align_ws_bytes(P, E) bytes for the counts.
size_t align_ws_bytes(int64_t P, int E);
// With wide_table (B = kWideBlockRows, E <= kWidePrepMaxExperts), the placement
// kernel also writes the expert-wide tile table (the layout launch_wide_prep
// writes), from the per-expert segment sizes it computes anyway.
hipError_t launch_align_ws(const int32_t* topk_ids, int64_t P, int E, int B, int32_t* sorted_ids,
                           int32_t* expert_ids, int32_t* total, int64_t max_padded, int32_t* hist,
                           hipStream_t stream, int32_t* wide_table = nullptr);

// Packed expert weights (see moe_pack_weights in moe.h): tiles of 256 rows,
// K stages of 64 bytes, one 16 KiB block per (expert, tile, stage).
constexpr int kPackRows = 256;
constexpr int kPackStageBytes = 64;
constexpr int kPackBlockBytes = kPackRows * kPackStageBytes;

__host__ __device__ inline int64_t packed_tiles(int64_t N, int silu) {
  return silu ? (N / 2 + kPackRows / 2 - 1) / (kPackRows / 2) : (N + kPackRows - 1) / kPackRows;
}
__host__ __device__ inline int64_t packed_kstages(int64_t K_elems, int elem_bytes) {
  return (K_elems * elem_bytes + kPackStageBytes - 1) / kPackStageBytes;
}

hipError_t launch_pack_weights(const void* w, int elem_bytes, int E, int64_t N, int64_t K, int silu,
                               void* packed, hipStream_t stream);

struct MoeGemmArgs {
  const void* A;
  int a_dtype;            // 0 f32, 1 bf16
  int64_t lda;
  int a_rows;             // 0 pair, 1 sorted
  int a_row_div;
  const void* B;          // [E, N, K] bf16, or packed (b_packed)
  int b_packed;
  int E;
  int64_t N, K;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* total;
  int64_t max_padded;
  int block_m;
  int64_t num_valid;
  const float* topk_weights;
  int epilogue;           // 0 none, 1 silu_mul
  void* C;
  int c_dtype;            // 0 f32, 1 bf16, 2 f16
  int64_t ldc;
  int c_rows;             // 0 pair, 1 sorted
  // int8 operands (a_dtype 3, B int8): exact int32 sums, then
  //   value = sum * a_scales[A row] * b_scales[e * N + n]
  const float* a_scales;  // indexed like A rows
  const float* b_scales;  // [E, N]
};

// MFMA tile kernel, block_m 64 or 128.
hipError_t launch_moe_gemm_tile(const MoeGemmArgs& a, hipStream_t stream);

// Expert-wide tiles (bf16 tokens and h, block_m 32): a tile table of
// wide_table_ints(max_padded) ints built from the alignment by
// launch_wide_prep (or by launch_align_ws itself), then one launch per GEMM
// (gate_up with SiLU*up into h in sorted order; down with the routing weight
// into pair rows).  Table: t[0] = number of tiles; tile j: t[1 + 3j] =
// expert, t[2 + 3j] = first block, t[3 + 3j] = blocks; an expert of n blocks
// gets ceil(n / kWideMaxBlocks) tiles, tile i of its t tiles starting at
// block first + floor(i * n / t).
#ifndef MOE_WIDE_MAXBLK
#define MOE_WIDE_MAXBLK 10
#endif
constexpr int kWideBlockRows = 32;
constexpr int kWideMaxBlocks = MOE_WIDE_MAXBLK;
constexpr int kWidePrepMaxExperts = 1024;
int64_t wide_table_ints(int64_t max_padded);
hipError_t launch_wide_prep(const int32_t* expert_ids, const int32_t* total, int E,
                            int64_t max_padded, int32_t* table, hipStream_t stream);
hipError_t launch_moe_gemm_wide(const MoeGemmArgs& a, const int32_t* table, hipStream_t stream);
// Weight-streaming kernel, block_m 16 or 32.
hipError_t launch_moe_gemm_stream(const MoeGemmArgs& a, hipStream_t stream);

// out[t, :] = sum_k y[t * topk + k, :]   (fp32 sum in the order k = 0 .. topk-1)
// y_dtype / out_dtype: 0 f32, 1 bf16 (out also 2 f16).
hipError_t launch_topk_reduce(const void* y, int y_dtype, int64_t T, int topk, int64_t H,
                              void* out, int out_dtype, hipStream_t stream);

// The layer after routing in one launch, for small problems
// (small_layer.hip): one workgroup per token.  H and I multiples of 8.
struct SmallLayerArgs {
  const void* x;
  int x_dtype;            // 0 f32, 1 bf16; out in the same dtype
  const int32_t* ids;     // [T * topk] routed experts, pair order
  const float* w;         // [T * topk] routing weights
  const void* w1;         // [E, 2I, H] bf16
  const void* w2;         // [E, H, I] bf16
  void* out;              // [T, H]
  int64_t T;
  int H, I, topk;
};
bool small_layer_fits(int64_t T, int H, int I, int E, int topk);
hipError_t launch_small_layer(const SmallLayerArgs& a, hipStream_t stream);

struct GmmI8Args {
  const int8_t* X;
  const int8_t* W;        // [E, N, K] int8, or packed (w_packed)
  int w_packed;
  const float* sx;
  const float* sw;
  const int32_t* offsets;
  void* Y;
  int64_t M, K, N;
  int E;
};

hipError_t launch_gmm_int8(const GmmI8Args& a, hipStream_t stream);

// Symmetric per-row int8 quantisation in float32: scale = max|row| / 127
// (1 for an all-zero row), q = clamp(rint(x / scale), -127, 127).  x dtype
// 0 f32 or 1 bf16, row stride ld elements.  With sorted_ids != nullptr only
// rows r < *total whose sorted_ids[r] < num_valid are processed (the valid
// rows of a sorted buffer); the others are left untouched.
hipError_t launch_quantize_rows(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld,
                                const int32_t* sorted_ids, const int32_t* total, int64_t num_valid,
                                int8_t* q, float* scales, hipStream_t stream);

}  // namespace moe

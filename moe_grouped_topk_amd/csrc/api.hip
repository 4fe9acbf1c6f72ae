// C ABI of the fused-MoE library: argument validation, workspace layout and
// the enqueue order of the layer.  Declarations and the contract of every
// entry point are in include/moe.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "moe.h"   // include/ is on the include path
#include "launch.hpp"

// Workspace of moe_forward_noalloc (see scratch_address below).
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of moe_forward_noalloc: a static device array, one copy per
// device, held until the process ends.  Its name is a host-side stand-in in
// host code; the device address comes from hipGetSymbolAddress, looked up once
// per device (with that device current) and kept.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array; null if HIP fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);   // racing first calls store the same
  return p;
}

// Shape and option checks of the routing step (pointers are checked by the caller).
int check_route_shape(int64_t T, int32_t E, int32_t topk, int32_t G, int32_t Kg, int32_t scoring) {
  if (T < 0) return MOE_ERR_SHAPE;
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (topk < 1 || topk > MOE_MAX_TOPK || topk > E) return MOE_ERR_SHAPE;
  if (G < 1 || G > 64 || E % G != 0) return MOE_ERR_CONFIG;
  if (Kg < 1 || Kg > G) return MOE_ERR_CONFIG;
  if ((int64_t)topk > (int64_t)Kg * (E / G)) return MOE_ERR_CONFIG;
  if (scoring != MOE_SCORING_SOFTMAX && scoring != MOE_SCORING_SIGMOID) return MOE_ERR_CONFIG;
  if (T * (int64_t)topk >= INT32_MAX) return MOE_ERR_SHAPE;
  return MOE_OK;
}

bool valid_block_m(int32_t b) { return b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

int64_t align_max_padded(int64_t P, int32_t E, int32_t B) {
  const int64_t nonempty = P < E ? P : E;
  const int64_t bound = P + nonempty * (B - 1);
  return (bound + B - 1) / B * B;
}

// wide: the call runs on the expert-wide tile kernel (block 32, packed allowed)
int check_gemm(const moe::MoeGemmArgs& a, bool wide = false) {
  if (!a.B || !a.total) return MOE_ERR_NULL;
  if (a.max_padded > 0 && (!a.A || !a.C || !a.sorted_ids || !a.expert_ids)) return MOE_ERR_NULL;
  if (a.a_dtype != MOE_DTYPE_F32 && a.a_dtype != MOE_DTYPE_BF16 && a.a_dtype != MOE_DTYPE_I8)
    return MOE_ERR_DTYPE;
  if (a.a_dtype == MOE_DTYPE_I8) {   // int8 tokens and weights (moe_forward_w8a8)
    if ((a.block_m < 64 && !wide) || !a.a_scales || !a.b_scales) return MOE_ERR_CONFIG;
    if (a.c_dtype != MOE_DTYPE_F32 && a.c_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
    if (a.K % 16 != 0 || a.lda % 16 != 0) return MOE_ERR_SHAPE;
    if (!aligned16(a.b_scales)) return MOE_ERR_SHAPE;
  }
  if (a.c_dtype != MOE_DTYPE_F32 && a.c_dtype != MOE_DTYPE_BF16 && a.c_dtype != MOE_DTYPE_F16)
    return MOE_ERR_DTYPE;
  if (a.epilogue != MOE_EPILOGUE_NONE && a.epilogue != MOE_EPILOGUE_SILU_MUL) return MOE_ERR_CONFIG;
  if (a.a_rows != MOE_ROWS_PAIR && a.a_rows != MOE_ROWS_SORTED) return MOE_ERR_CONFIG;
  if (a.c_rows != MOE_ROWS_PAIR && a.c_rows != MOE_ROWS_SORTED) return MOE_ERR_CONFIG;
  if (!valid_block_m(a.block_m)) return MOE_ERR_CONFIG;
  if (a.block_m == 256 && a.a_dtype == MOE_DTYPE_F32) return MOE_ERR_CONFIG;
  if (a.a_rows == MOE_ROWS_PAIR && a.a_row_div < 1) return MOE_ERR_CONFIG;
  if (a.b_packed && ((a.block_m < 64 && !wide) || a.a_dtype == MOE_DTYPE_F32))
    return MOE_ERR_CONFIG;
  if (a.E < 1 || a.N < 16 || a.K < 8 || a.K % 8 != 0) return MOE_ERR_SHAPE;
  const int64_t nout = a.epilogue == MOE_EPILOGUE_SILU_MUL ? a.N / 2 : a.N;
  if (a.epilogue == MOE_EPILOGUE_SILU_MUL ? (a.N % 32 != 0) : (a.N % 16 != 0)) return MOE_ERR_SHAPE;
  if (a.lda < a.K || a.lda % 8 != 0) return MOE_ERR_SHAPE;
  if (a.ldc < nout || a.ldc % 8 != 0) return MOE_ERR_SHAPE;
  if (a.num_valid < 0 || a.num_valid >= INT32_MAX) return MOE_ERR_SHAPE;
  if (a.max_padded < 0 || a.max_padded >= INT32_MAX) return MOE_ERR_SHAPE;
  if (a.max_padded > 0 && (!aligned16(a.A) || !aligned16(a.B) || !aligned16(a.C)))
    return MOE_ERR_SHAPE;
  // grid sizes stay inside 32-bit workgroup counts
  const int64_t ntile = (nout + 63) / 64 + 1;
  if ((a.max_padded / a.block_m) * ntile >= INT32_MAX) return MOE_ERR_SHAPE;
  return MOE_OK;
}

int enqueue_gemm(const moe::MoeGemmArgs& a, hipStream_t s) {
  if (a.max_padded == 0) return MOE_OK;
  const hipError_t err = a.block_m <= 32 ? moe::launch_moe_gemm_stream(a, s)
                                         : moe::launch_moe_gemm_tile(a, s);
  return hip_status(err);
}

// Packed weights run on the tile kernels (block_m >= 64) or, with bf16 tokens,
// on the expert-wide tiles (block 32); with few rows per expert the tile
// kernels skip the MFMAs of empty token columns and stream weights.
// (wide: the bf16 layer may take the expert-wide tiles; the int8 layer may not)
int choose_block_m(int64_t T, int32_t E, int32_t topk, int32_t x_dtype, int32_t w_layout,
                   bool wide = true) {
  const double avg = (double)T * topk / (double)E;   // pairs per expert
  // bf16 tokens, many pairs per expert: one tile per expert and 256 weight
  // rows streams every weight slice once (prefill T = 4096, E = 128: layer
  // 465 us against 504 us on 256 x 128 tiles at block 128, same bits)
  if (wide && avg >= 96.0 && x_dtype == MOE_DTYPE_BF16 && E <= moe::kWidePrepMaxExperts)
    return 32;
  // bf16 tokens take the direct-to-LDS tile kernels at any size (decode
  // T = 16 on plain weights: 1.59 ms at block 64 against 2.40 ms with the
  // weight-streaming kernel at block 16); f32 tokens with plain weights keep
  // the streaming kernel for few pairs per expert
  const bool tile = w_layout == MOE_WEIGHTS_PACKED || x_dtype == MOE_DTYPE_BF16;
  if (avg < 8.0 && !tile) return 16;
  if (avg < 24.0 && !tile) return 32;
  if (avg < 96.0) return 64;
  return 128;   // 256 x 128 tiles, two workgroups per CU: measured ahead of 256 x 256
}

bool valid_layout(int32_t l) { return l == MOE_WEIGHTS_PLAIN || l == MOE_WEIGHTS_PACKED; }

struct ForwardLayout {
  size_t w, ids, sorted, eids, total, hist, h, y, table, bytes;
  int64_t max_padded;
  int block_m;
  bool small;   // the layer after routing runs as one launch (small_layer.hip)
  bool wide;    // bf16 tokens at block 32: expert-wide tiles from a tile table
};

bool use_wide(int32_t block_m, int32_t x_dtype, int32_t E) {
  return block_m == 32 && x_dtype == MOE_DTYPE_BF16 && E <= moe::kWidePrepMaxExperts;
}

// Small layers with plain weights and the automatic block size skip the
// alignment and run both GEMMs and the sum in one launch after routing.
bool use_small_layer(int64_t T, int32_t H, int32_t I, int32_t E, int32_t topk, int32_t block_m,
                     int32_t w_layout) {
  return block_m == 0 && w_layout == MOE_WEIGHTS_PLAIN && moe::small_layer_fits(T, H, I, E, topk);
}

ForwardLayout forward_layout(int64_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                             int32_t block_m, int32_t x_dtype, int32_t w_layout) {
  ForwardLayout L{};
  L.block_m = block_m ? block_m : choose_block_m(T, E, topk, x_dtype, w_layout);
  const int64_t P = T * topk;
  L.max_padded = align_max_padded(P, E, L.block_m);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = round_up(off + bytes, 256); return o; };
  L.w = take(sizeof(float) * (size_t)P);
  L.ids = take(sizeof(int32_t) * (size_t)P);
  L.sorted = take(sizeof(int32_t) * (size_t)L.max_padded);
  L.eids = take(sizeof(int32_t) * (size_t)(L.max_padded / L.block_m));
  L.total = take(sizeof(int32_t));
  L.hist = take(moe::align_ws_bytes(P, E));
  L.h = take(2 * (size_t)L.max_padded * (size_t)I);
  L.y = take((x_dtype == MOE_DTYPE_F32 ? 4 : 2) * (size_t)P * (size_t)H);
  L.small = use_small_layer(T, H, I, E, topk, block_m, w_layout);
  L.wide = !L.small && use_wide(L.block_m, x_dtype, E);
  if (L.wide) L.table = take(sizeof(int32_t) * (size_t)moe::wide_table_ints(L.max_padded));
  L.bytes = off;
  return L;
}

// Workspace of moe_forward_w8a8 (256-byte aligned pieces).
struct W8a8Layout {
  size_t w, ids, sorted, eids, total, hist, xq, sx, h, hq, sh, y, table, bytes;
  int64_t max_padded;
  int block_m;
  bool wide;    // bf16 x at block 32: expert-wide int8 tiles from a tile table
};

W8a8Layout w8a8_layout(int64_t T, int32_t H, int32_t I, int32_t E, int32_t topk, int32_t block_m,
                       int32_t x_dtype) {
  W8a8Layout L{};
  L.block_m = block_m ? block_m : choose_block_m(T, E, topk, x_dtype, MOE_WEIGHTS_PACKED);
  const int64_t P = T * topk;
  L.max_padded = align_max_padded(P, E, L.block_m);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = round_up(off + bytes, 256); return o; };
  L.w = take(sizeof(float) * (size_t)P);
  L.ids = take(sizeof(int32_t) * (size_t)P);
  L.sorted = take(sizeof(int32_t) * (size_t)L.max_padded);
  L.eids = take(sizeof(int32_t) * (size_t)(L.max_padded / L.block_m));
  L.total = take(sizeof(int32_t));
  L.hist = take(moe::align_ws_bytes(P, E));
  L.xq = take((size_t)T * (size_t)H);
  L.sx = take(sizeof(float) * (size_t)T);
  L.h = take(2 * (size_t)L.max_padded * (size_t)I);   // bf16
  L.hq = take((size_t)L.max_padded * (size_t)I);
  L.sh = take(sizeof(float) * (size_t)L.max_padded);
  L.y = take((x_dtype == MOE_DTYPE_F32 ? 4 : 2) * (size_t)P * (size_t)H);
  L.wide = use_wide(L.block_m, x_dtype, E);
  if (L.wide) L.table = take(sizeof(int32_t) * (size_t)moe::wide_table_ints(L.max_padded));
  L.bytes = off;
  return L;
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer argument";
    case MOE_ERR_SHAPE: return "size out of range or inconsistent";
    case MOE_ERR_CONFIG: return "invalid option or option combination";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int moe_route(const float* gating, int64_t T, int32_t E, int32_t topk, int32_t num_expert_group,
              int32_t topk_group, int32_t scoring, int32_t renormalize,
              float routed_scaling_factor, float* topk_weights, int32_t* topk_ids,
              void* stream) {
  const int st = check_route_shape(T, E, topk, num_expert_group, topk_group, scoring);
  if (st != MOE_OK) return st;
  if (T > 0 && (!gating || !topk_weights || !topk_ids)) return MOE_ERR_NULL;
  return hip_status(moe::launch_route(gating, T, E, topk, num_expert_group, topk_group, scoring,
                                      renormalize ? 1 : 0, routed_scaling_factor, topk_weights,
                                      topk_ids, as_stream(stream)));
}

int64_t moe_align_max_padded(int64_t num_pairs, int32_t E, int32_t block_m) {
  if (num_pairs < 0 || E < 1 || block_m < 1) return -1;
  return align_max_padded(num_pairs, E, block_m);
}

size_t moe_align_workspace_size(int64_t num_pairs, int32_t E) {
  if (num_pairs < 0 || num_pairs >= INT32_MAX || E < 1 || E > MOE_MAX_EXPERTS) return 0;
  return moe::align_ws_bytes(num_pairs, E);
}

int moe_align_block_size(const int32_t* topk_ids, int64_t num_pairs, int32_t E, int32_t block_m,
                         int32_t* sorted_token_ids, int32_t* expert_ids,
                         int32_t* num_tokens_post_padded, int64_t max_padded, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!num_tokens_post_padded) return MOE_ERR_NULL;
  if (num_pairs > 0 && !topk_ids) return MOE_ERR_NULL;
  // empty buffers (capacity 0) may come with null pointers
  if (max_padded > 0 && !sorted_token_ids) return MOE_ERR_NULL;
  if (block_m > 0 && max_padded / block_m > 0 && !expert_ids) return MOE_ERR_NULL;
  if (num_pairs < 0 || num_pairs >= INT32_MAX) return MOE_ERR_SHAPE;
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (block_m < 1 || block_m > 1024) return MOE_ERR_CONFIG;
  if (max_padded < align_max_padded(num_pairs, E, block_m) || max_padded >= INT32_MAX)
    return MOE_ERR_SHAPE;
  if (ws) {
    if (ws_bytes < moe::align_ws_bytes(num_pairs, E) || !aligned16(ws)) return MOE_ERR_WORKSPACE;
    return hip_status(moe::launch_align_ws(topk_ids, num_pairs, E, block_m, sorted_token_ids,
                                           expert_ids, num_tokens_post_padded, max_padded,
                                           reinterpret_cast<int32_t*>(ws), as_stream(stream)));
  }
  return hip_status(moe::launch_align(topk_ids, num_pairs, E, block_m, sorted_token_ids,
                                      expert_ids, num_tokens_post_padded, max_padded,
                                      as_stream(stream)));
}

size_t moe_packed_weights_size(int32_t dtype, int32_t E, int64_t N, int64_t K, int32_t epilogue) {
  if (E < 1 || E > MOE_MAX_EXPERTS) return 0;
  if (epilogue != MOE_EPILOGUE_NONE && epilogue != MOE_EPILOGUE_SILU_MUL) return 0;
  int elem;
  if (dtype == MOE_DTYPE_BF16) {
    if (N < 16 || K < 8 || K % 8 != 0) return 0;
    if (epilogue == MOE_EPILOGUE_SILU_MUL ? (N % 32 != 0) : (N % 16 != 0)) return 0;
    elem = 2;
  } else if (dtype == MOE_DTYPE_I8) {
    if (N < 16 || K < 16 || K % 16 != 0 || K > 131072) return 0;
    if (epilogue == MOE_EPILOGUE_SILU_MUL ? (N % 32 != 0) : (N % 16 != 0)) return 0;
    elem = 1;
  } else {
    return 0;
  }
  const int silu = epilogue == MOE_EPILOGUE_SILU_MUL;
  return (size_t)E * (size_t)moe::packed_tiles(N, silu) * (size_t)moe::packed_kstages(K, elem) *
         (size_t)moe::kPackBlockBytes;
}

int moe_pack_weights(const void* w, int32_t dtype, int32_t E, int64_t N, int64_t K, int32_t epilogue,
                     void* packed, size_t packed_bytes, void* stream) {
  if (epilogue != MOE_EPILOGUE_NONE && epilogue != MOE_EPILOGUE_SILU_MUL) return MOE_ERR_CONFIG;
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_I8) return MOE_ERR_DTYPE;
  const size_t need = moe_packed_weights_size(dtype, E, N, K, epilogue);
  if (need == 0) return MOE_ERR_SHAPE;
  if (!w || !packed) return MOE_ERR_NULL;
  if (packed_bytes < need) return MOE_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_pack_weights(w, dtype == MOE_DTYPE_I8 ? 1 : 2, E, N, K,
                                             epilogue == MOE_EPILOGUE_SILU_MUL, packed,
                                             as_stream(stream)));
}

int moe_grouped_gemm(const void* A, int32_t a_dtype, int64_t lda, int32_t a_rows, int32_t a_row_div,
                     const void* B, int32_t b_layout, int32_t E, int64_t N, int64_t K,
                     const int32_t* sorted_token_ids, const int32_t* expert_ids,
                     const int32_t* num_tokens_post_padded, int64_t max_padded, int32_t block_m,
                     int64_t num_valid_pairs, const float* topk_weights, int32_t epilogue, void* C,
                     int32_t c_dtype, int64_t ldc, int32_t c_rows, void* stream) {
  moe::MoeGemmArgs a{};
  a.A = A; a.a_dtype = a_dtype; a.lda = lda; a.a_rows = a_rows;
  a.a_row_div = a_row_div < 1 ? 1 : a_row_div;
  if (a_rows == MOE_ROWS_PAIR && a_row_div < 1) return MOE_ERR_CONFIG;
  if (!valid_layout(b_layout)) return MOE_ERR_CONFIG;
  if (a_dtype == MOE_DTYPE_I8) return MOE_ERR_DTYPE;   // int8 runs through moe_forward_w8a8
  a.B = B; a.b_packed = b_layout == MOE_WEIGHTS_PACKED; a.E = E; a.N = N; a.K = K;
  a.sorted_ids = sorted_token_ids; a.expert_ids = expert_ids; a.total = num_tokens_post_padded;
  a.max_padded = max_padded; a.block_m = block_m; a.num_valid = num_valid_pairs;
  a.topk_weights = topk_weights; a.epilogue = epilogue;
  a.C = C; a.c_dtype = c_dtype; a.ldc = ldc; a.c_rows = c_rows;
  const int st = check_gemm(a);
  if (st != MOE_OK) return st;
  return enqueue_gemm(a, as_stream(stream));
}

int64_t moe_wide_tile_table_size(int64_t max_padded) {
  if (max_padded < 0 || max_padded % 32 != 0) return -1;
  return moe::wide_table_ints(max_padded);
}

int moe_wide_tile_table(const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                        int32_t E, int64_t max_padded, int32_t* table, int64_t table_ints,
                        void* stream) {
  if (!num_tokens_post_padded || !table) return MOE_ERR_NULL;
  if (max_padded > 0 && !expert_ids) return MOE_ERR_NULL;
  if (E < 1 || E > moe::kWidePrepMaxExperts) return MOE_ERR_CONFIG;
  if (max_padded < 0 || max_padded % 32 != 0 || max_padded >= INT32_MAX) return MOE_ERR_SHAPE;
  if (table_ints < moe::wide_table_ints(max_padded)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_wide_prep(expert_ids, num_tokens_post_padded, E, max_padded,
                                          table, as_stream(stream)));
}

int moe_grouped_gemm_wide(const void* A, int32_t a_dtype, int64_t lda, int32_t a_rows,
                          int32_t a_row_div, const void* B, int32_t b_layout, int32_t E, int64_t N,
                          int64_t K, const int32_t* sorted_token_ids, const int32_t* expert_ids,
                          const int32_t* num_tokens_post_padded, int64_t max_padded,
                          const int32_t* tile_table, int64_t num_valid_pairs,
                          const float* topk_weights, int32_t epilogue, void* C, int32_t c_dtype,
                          int64_t ldc, int32_t c_rows, void* stream) {
  moe::MoeGemmArgs a{};
  a.A = A; a.a_dtype = a_dtype; a.lda = lda; a.a_rows = a_rows;
  a.a_row_div = a_row_div < 1 ? 1 : a_row_div;
  if (a_rows == MOE_ROWS_PAIR && a_row_div < 1) return MOE_ERR_CONFIG;
  if (!valid_layout(b_layout)) return MOE_ERR_CONFIG;
  if (a_dtype != MOE_DTYPE_BF16 || c_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (epilogue == MOE_EPILOGUE_SILU_MUL && topk_weights) return MOE_ERR_CONFIG;
  if (E > moe::kWidePrepMaxExperts) return MOE_ERR_CONFIG;
  a.B = B; a.b_packed = b_layout == MOE_WEIGHTS_PACKED; a.E = E; a.N = N; a.K = K;
  a.sorted_ids = sorted_token_ids; a.expert_ids = expert_ids; a.total = num_tokens_post_padded;
  a.max_padded = max_padded; a.block_m = 32; a.num_valid = num_valid_pairs;
  a.topk_weights = topk_weights; a.epilogue = epilogue;
  a.C = C; a.c_dtype = c_dtype; a.ldc = ldc; a.c_rows = c_rows;
  const int st = check_gemm(a, true);
  if (st != MOE_OK) return st;
  if (max_padded == 0) return MOE_OK;
  if (!tile_table) return MOE_ERR_NULL;
  return hip_status(moe::launch_moe_gemm_wide(a, tile_table, as_stream(stream)));
}

int32_t moe_forward_block_m(int64_t T, int32_t E, int32_t topk, int32_t x_dtype, int32_t w_layout) {
  if (T < 0 || E < 1 || topk < 1) return -1;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return -1;
  if (!valid_layout(w_layout)) return -1;
  return choose_block_m(T, E, topk, x_dtype, w_layout);
}

size_t moe_forward_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                                  int32_t block_m) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || topk < 1) return 0;
  if (block_m != 0 && !valid_block_m(block_m)) return 0;
  // the automatic block size can depend on x's dtype and the weight layout: cover all
  size_t most = 0;
  for (int32_t dt : {MOE_DTYPE_BF16, MOE_DTYPE_F32})
    for (int32_t wl : {MOE_WEIGHTS_PLAIN, MOE_WEIGHTS_PACKED}) {
      const size_t b = forward_layout(T, H, I, E, topk, block_m, dt, wl).bytes;
      most = b > most ? b : most;
    }
  return most;
}

}  // extern "C"

namespace {

// moe_forward's work on a caller's workspace (ws, ws_bytes), or, with
// use_scratch set, on this device's static scratch array (ws is ignored).
int forward_impl(const void* x, int32_t x_dtype, const float* gating, const void* w1,
                 const void* w2, int32_t w_layout, int64_t T, int32_t H, int32_t I, int32_t E,
                 int32_t topk, int32_t num_expert_group, int32_t topk_group, int32_t scoring,
                 int32_t renormalize, float routed_scaling_factor, int32_t block_m, void* out,
                 float* topk_weights_out, int32_t* topk_ids_out, void* ws, size_t ws_bytes,
                 bool use_scratch, void* stream) {
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (block_m != 0 && !valid_block_m(block_m)) return MOE_ERR_CONFIG;
  if (!valid_layout(w_layout)) return MOE_ERR_CONFIG;
  const bool packed = w_layout == MOE_WEIGHTS_PACKED;
  if (packed && (x_dtype != MOE_DTYPE_BF16 ||
                 (block_m != 0 && block_m < 64 && !use_wide(block_m, x_dtype, E))))
    return MOE_ERR_CONFIG;
  if (H < 16 || H % 16 != 0 || I < 16 || I % 16 != 0) return MOE_ERR_SHAPE;
  int st = check_route_shape(T, E, topk, num_expert_group, topk_group, scoring);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !gating || !w1 || !w2 || !out) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(out)) return MOE_ERR_SHAPE;
  const ForwardLayout L = forward_layout(T, H, I, E, topk, block_m, x_dtype, w_layout);
  if (use_scratch) {
    if (L.bytes > kScratchBytes) return MOE_ERR_WORKSPACE;
    ws = scratch_address();
    ws_bytes = kScratchBytes;
    if (!ws) return MOE_ERR_HIP;
  }
  if (!ws || ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_WORKSPACE;
  if (L.max_padded >= INT32_MAX) return MOE_ERR_SHAPE;

  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  float* w = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(base + L.w);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + L.ids);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(base + L.eids);
  int32_t* total = reinterpret_cast<int32_t*>(base + L.total);
  void* h = base + L.h;
  void* y = base + L.y;   // per-pair down-projection rows, in x's dtype
  hipStream_t s = as_stream(stream);
  const int64_t P = T * topk;

  hipError_t err = moe::launch_route(gating, T, E, topk, num_expert_group, topk_group, scoring,
                                     renormalize ? 1 : 0, routed_scaling_factor, w, ids, s);
  if (err != hipSuccess) return MOE_ERR_HIP;
  if (L.small) {
    moe::SmallLayerArgs a{};
    a.x = x; a.x_dtype = x_dtype == MOE_DTYPE_F32 ? 0 : 1; a.ids = ids; a.w = w;
    a.w1 = w1; a.w2 = w2; a.out = out; a.T = T; a.H = H; a.I = I; a.topk = topk;
    return hip_status(moe::launch_small_layer(a, s));
  }
  int32_t* table = L.wide ? reinterpret_cast<int32_t*>(base + L.table) : nullptr;
  err = moe::launch_align_ws(ids, P, E, L.block_m, sorted, eids, total, L.max_padded,
                             reinterpret_cast<int32_t*>(base + L.hist), s, table);
  if (err != hipSuccess) return MOE_ERR_HIP;

  moe::MoeGemmArgs g1{};
  g1.A = x; g1.a_dtype = x_dtype; g1.lda = H; g1.a_rows = MOE_ROWS_PAIR; g1.a_row_div = topk;
  g1.B = w1; g1.b_packed = packed; g1.E = E; g1.N = 2 * (int64_t)I; g1.K = H;
  g1.sorted_ids = sorted; g1.expert_ids = eids; g1.total = total; g1.max_padded = L.max_padded;
  g1.block_m = L.block_m; g1.num_valid = P; g1.topk_weights = nullptr;
  g1.epilogue = MOE_EPILOGUE_SILU_MUL; g1.C = h; g1.c_dtype = MOE_DTYPE_BF16; g1.ldc = I;
  g1.c_rows = MOE_ROWS_SORTED;
  st = check_gemm(g1, L.wide);
  if (st != MOE_OK) return st;

  moe::MoeGemmArgs g2 = g1;
  g2.A = h; g2.a_dtype = MOE_DTYPE_BF16; g2.lda = I; g2.a_rows = MOE_ROWS_SORTED; g2.a_row_div = 1;
  g2.B = w2; g2.N = H; g2.K = I; g2.topk_weights = w; g2.epilogue = MOE_EPILOGUE_NONE;
  g2.C = y; g2.c_dtype = x_dtype; g2.ldc = H; g2.c_rows = MOE_ROWS_PAIR;
  st = check_gemm(g2, L.wide);
  if (st != MOE_OK) return st;

  if (L.wide) {   // the alignment wrote the tile table
    err = moe::launch_moe_gemm_wide(g1, table, s);
    if (err == hipSuccess) err = moe::launch_moe_gemm_wide(g2, table, s);
    if (err != hipSuccess) return hip_status(err);
  } else {
    st = enqueue_gemm(g1, s);
    if (st == MOE_OK) st = enqueue_gemm(g2, s);
    if (st != MOE_OK) return st;
  }
  return hip_status(moe::launch_topk_reduce(y, x_dtype, T, topk, H, out, x_dtype, s));
}

}  // namespace

extern "C" {

int moe_forward(const void* x, int32_t x_dtype, const float* gating, const void* w1, const void* w2,
                int32_t w_layout, int64_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                int32_t num_expert_group, int32_t topk_group, int32_t scoring,
                int32_t renormalize, float routed_scaling_factor, int32_t block_m, void* out,
                float* topk_weights_out, int32_t* topk_ids_out, void* ws, size_t ws_bytes,
                void* stream) {
  return forward_impl(x, x_dtype, gating, w1, w2, w_layout, T, H, I, E, topk, num_expert_group,
                      topk_group, scoring, renormalize, routed_scaling_factor, block_m, out,
                      topk_weights_out, topk_ids_out, ws, ws_bytes, false, stream);
}

int moe_forward_noalloc(const void* x, int32_t x_dtype, const float* gating, const void* w1,
                        const void* w2, int32_t w_layout, int64_t T, int32_t H, int32_t I,
                        int32_t E, int32_t topk, int32_t num_expert_group, int32_t topk_group,
                        int32_t scoring, int32_t renormalize, float routed_scaling_factor,
                        int32_t block_m, void* out, float* topk_weights_out,
                        int32_t* topk_ids_out, void* stream) {
  return forward_impl(x, x_dtype, gating, w1, w2, w_layout, T, H, I, E, topk, num_expert_group,
                      topk_group, scoring, renormalize, routed_scaling_factor, block_m, out,
                      topk_weights_out, topk_ids_out, nullptr, 0, true, stream);
}

int moe_quantize_rows(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int64_t ld,
                      int8_t* q, float* scales, void* stream) {
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (rows < 0 || cols < 8 || cols % 8 != 0 || ld < cols || ld % 8 != 0) return MOE_ERR_SHAPE;
  if (rows >= ((int64_t)1 << 40)) return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(q)) return MOE_ERR_SHAPE;
  return hip_status(moe::launch_quantize_rows(x, x_dtype, rows, cols, ld, nullptr, nullptr, 0, q,
                                              scales, as_stream(stream)));
}

size_t moe_forward_w8a8_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                                       int32_t block_m) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || topk < 1) return 0;
  if (block_m != 0 && (!valid_block_m(block_m) || (block_m < 64 && block_m != 32))) return 0;
  size_t most = 0;
  for (int32_t dt : {MOE_DTYPE_BF16, MOE_DTYPE_F32}) {
    const size_t b = w8a8_layout(T, H, I, E, topk, block_m, dt).bytes;
    most = b > most ? b : most;
  }
  return most;
}

int moe_forward_w8a8(const void* x, int32_t x_dtype, const float* gating, const int8_t* w1q,
                     const float* w1_scales, const int8_t* w2q, const float* w2_scales,
                     int32_t w_layout, int64_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                     int32_t num_expert_group, int32_t topk_group, int32_t scoring,
                     int32_t renormalize, float routed_scaling_factor, int32_t block_m, void* out,
                     float* topk_weights_out, int32_t* topk_ids_out, void* ws, size_t ws_bytes,
                     void* stream) {
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (!valid_layout(w_layout)) return MOE_ERR_CONFIG;
  if (block_m != 0 &&
      (!valid_block_m(block_m) || (block_m < 64 && !use_wide(block_m, x_dtype, E))))
    return MOE_ERR_CONFIG;
  if (H < 16 || H % 16 != 0 || I < 16 || I % 16 != 0 || H > 131072 || I > 131072)
    return MOE_ERR_SHAPE;
  int st = check_route_shape(T, E, topk, num_expert_group, topk_group, scoring);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !gating || !w1q || !w2q || !w1_scales || !w2_scales || !out) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w1q) || !aligned16(w2q) || !aligned16(out) ||
      !aligned16(w1_scales) || !aligned16(w2_scales))
    return MOE_ERR_SHAPE;
  const W8a8Layout L = w8a8_layout(T, H, I, E, topk, block_m, x_dtype);
  if (!ws || ws_bytes < L.bytes) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_WORKSPACE;
  if (L.max_padded >= INT32_MAX) return MOE_ERR_SHAPE;

  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  float* w = topk_weights_out ? topk_weights_out : reinterpret_cast<float*>(base + L.w);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + L.ids);
  int32_t* sorted = reinterpret_cast<int32_t*>(base + L.sorted);
  int32_t* eids = reinterpret_cast<int32_t*>(base + L.eids);
  int32_t* total = reinterpret_cast<int32_t*>(base + L.total);
  int8_t* xq = reinterpret_cast<int8_t*>(base + L.xq);
  float* sx = reinterpret_cast<float*>(base + L.sx);
  void* h = base + L.h;   // gate_up output, bf16, quantised per row below
  int8_t* hq = reinterpret_cast<int8_t*>(base + L.hq);
  float* sh = reinterpret_cast<float*>(base + L.sh);
  void* y = base + L.y;
  hipStream_t s = as_stream(stream);
  const int64_t P = T * topk;
  const bool packed = w_layout == MOE_WEIGHTS_PACKED;

  moe::MoeGemmArgs g1{};
  g1.A = xq; g1.a_dtype = MOE_DTYPE_I8; g1.lda = H; g1.a_rows = MOE_ROWS_PAIR; g1.a_row_div = topk;
  g1.a_scales = sx; g1.B = w1q; g1.b_packed = packed; g1.b_scales = w1_scales;
  g1.E = E; g1.N = 2 * (int64_t)I; g1.K = H;
  g1.sorted_ids = sorted; g1.expert_ids = eids; g1.total = total; g1.max_padded = L.max_padded;
  g1.block_m = L.block_m; g1.num_valid = P; g1.topk_weights = nullptr;
  g1.epilogue = MOE_EPILOGUE_SILU_MUL; g1.C = h; g1.c_dtype = MOE_DTYPE_BF16; g1.ldc = I;
  g1.c_rows = MOE_ROWS_SORTED;
  st = check_gemm(g1, L.wide);
  if (st != MOE_OK) return st;
  moe::MoeGemmArgs g2 = g1;
  g2.A = hq; g2.lda = I; g2.a_rows = MOE_ROWS_SORTED; g2.a_row_div = 1; g2.a_scales = sh;
  g2.B = w2q; g2.b_scales = w2_scales; g2.N = H; g2.K = I; g2.topk_weights = w;
  g2.epilogue = MOE_EPILOGUE_NONE; g2.C = y; g2.c_dtype = x_dtype; g2.ldc = H;
  g2.c_rows = MOE_ROWS_PAIR;
  st = check_gemm(g2, L.wide);
  if (st != MOE_OK) return st;

  // routing also quantises each token's x row as it loads it (one wave per
  // token for both)
  moe::RouteExtra rx{x, x_dtype == MOE_DTYPE_BF16 ? 1 : 0, H, xq, sx, nullptr, 0};
  hipError_t err = moe::launch_route(gating, T, E, topk, num_expert_group, topk_group, scoring,
                                     renormalize ? 1 : 0, routed_scaling_factor, w, ids, s, &rx);
  if (err != hipSuccess) return MOE_ERR_HIP;
  int32_t* table = L.wide ? reinterpret_cast<int32_t*>(base + L.table) : nullptr;
  err = moe::launch_align_ws(ids, P, E, L.block_m, sorted, eids, total, L.max_padded,
                             reinterpret_cast<int32_t*>(base + L.hist), s, table);
  if (err != hipSuccess) return MOE_ERR_HIP;
  st = L.wide ? hip_status(moe::launch_moe_gemm_wide(g1, table, s)) : enqueue_gemm(g1, s);
  if (st != MOE_OK) return st;
  err = moe::launch_quantize_rows(h, MOE_DTYPE_BF16, L.max_padded, I, I, sorted, total, P, hq, sh, s);
  if (err != hipSuccess) return MOE_ERR_HIP;
  st = L.wide ? hip_status(moe::launch_moe_gemm_wide(g2, table, s)) : enqueue_gemm(g2, s);
  if (st != MOE_OK) return st;
  return hip_status(moe::launch_topk_reduce(y, x_dtype, T, topk, H, out, x_dtype, s));
}

int gmm_int8(const int8_t* input, const int8_t* weights, int32_t w_layout, const float* scales_x,
             const float* scales_w, const int32_t* expert_offsets, const int32_t* expert_sizes,
             void* output, int64_t M, int64_t K, int64_t N, int32_t E, void* stream) {
  (void)expert_sizes;   // the offsets decide; sizes are redundant
  if (M < 0 || M >= INT32_MAX / 2) return MOE_ERR_SHAPE;
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_SHAPE;
  if (K < 16 || K % 16 != 0 || K > 131072) return MOE_ERR_SHAPE;
  if (N < 16 || N % 16 != 0) return MOE_ERR_SHAPE;
  if (!valid_layout(w_layout)) return MOE_ERR_CONFIG;
  if (!weights || !scales_w || !expert_offsets) return MOE_ERR_NULL;
  if (M > 0 && (!input || !scales_x || !output)) return MOE_ERR_NULL;
  if (M == 0) return MOE_OK;
  if (!aligned16(input) || !aligned16(weights) || !aligned16(scales_w) || !aligned16(output))
    return MOE_ERR_SHAPE;
  const int64_t grid = ((M + 127) / 128 + E) * ((N + 127) / 128);
  if (grid >= INT32_MAX) return MOE_ERR_SHAPE;
  moe::GmmI8Args a{input, weights, w_layout == MOE_WEIGHTS_PACKED, scales_x, scales_w, expert_offsets,
                   output, M, K, N, E};
  return hip_status(moe::launch_gmm_int8(a, as_stream(stream)));
}

}  // extern "C"

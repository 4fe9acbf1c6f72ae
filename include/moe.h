/*
 * moe.h - C ABI of the MI355X (gfx950) fused Mixture-of-Experts forward path.
 *
 * Sources of the operations (cited by tag below):
 *   [P1]  DatenLord, "From loops to fusion: the Fused MoE operator, Part 3"
 *         (community.aijishu.com/a/1060000000523566), sections 01 and 03.
 *   [GTK] "GroupedTopK operator optimisation primer" (blog.freezetheflame.cc),
 *         sections 二 (interface), 三 (3.1-3.6 semantics), 七 (shortcut),
 *         八 (top-k pitfalls).
 *   [MSG] mini-sglang handbook, "MoE and fused MoE"
 *         (anrans.github.io/ai-infra-handbooks/minisgl/perf/moe/), sections
 *         路由 (select_experts), fused MoE (moe_align_block_size,
 *         fused_moe_kernel, FusedMoeBackend.forward), 练习 (exercise 3).
 *   [GMM] low-precision grouped GEMM article (www.pwwt.cn/news/5863887/),
 *         sections 2.1 (definition), 3.1 (interface), 3.4 (layout), 5.3.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is DEVICE memory owned by the caller, unless the
 *     argument says otherwise.  The library never frees or keeps them.
 *   - Tensors are dense and row-major.  Expert weights are [E, N, K] with K
 *     contiguous ([GMM] 3.4).  bf16 means IEEE bfloat16 bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on that stream; none synchronises the
 *     host, so device-side totals (e.g. the padded length) stay on the device.
 *   - Arguments are validated on the host before anything is enqueued.  On an
 *     error nothing is launched and a negative MOE_ERR_* code is returned;
 *     MOE_ERR_HIP reports a failed launch (hipGetLastError).  No C++
 *     exception crosses this boundary.  Calls are reentrant; calls that
 *     write the same buffers must be ordered by the caller (same stream, or
 *     events).
 *   - Process-wide state, all of it set once and never freed:
 *       * each kernel's dynamic-LDS limit is raised on its first launch on a
 *         device that needs more than 64 KiB (again only if a later launch
 *         needs more), with a table of the limits raised;
 *       * the compute-unit count of each device (it sizes the persistent
 *         grid of the expert-wide GEMMs), read on its first use there;
 *       * the static scratch of moe_forward_noalloc (one array per device,
 *         its address looked up once per device).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define MOE_OK             0
#define MOE_ERR_NULL      -1   /* a required pointer is NULL               */
#define MOE_ERR_SHAPE     -2   /* a size is out of range or inconsistent   */
#define MOE_ERR_CONFIG    -3   /* an option value or combination is invalid */
#define MOE_ERR_DTYPE     -4   /* unsupported dtype code                   */
#define MOE_ERR_WORKSPACE -5   /* workspace missing or too small           */
#define MOE_ERR_HIP       -6   /* the HIP runtime reported a launch error  */

/* ---- enumerations ------------------------------------------------------ */
#define MOE_DTYPE_F32   0
#define MOE_DTYPE_BF16  1
#define MOE_DTYPE_F16   2
#define MOE_DTYPE_I8    3   /* int8 (packing, quantisation and the int8 paths only) */

#define MOE_SCORING_SOFTMAX 0
#define MOE_SCORING_SIGMOID 1

#define MOE_EPILOGUE_NONE     0   /* C = A_row . B[e]^T                      */
#define MOE_EPILOGUE_SILU_MUL 1   /* C = silu(A.Bgate^T) * (A.Bup^T)         */

#define MOE_ROWS_PAIR   0   /* row index = pair index (token*topk + k)      */
#define MOE_ROWS_SORTED 1   /* row index = position in sorted_token_ids     */

#define MOE_WEIGHTS_PLAIN  0   /* [E, N, K], K contiguous                    */
#define MOE_WEIGHTS_PACKED 1   /* written by moe_pack_weights (see there)    */

/* Largest supported sizes (validated; MOE_ERR_SHAPE beyond them). */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK    64

/* Human-readable name of a status code (static storage, never NULL). */
MOE_API const char* moe_status_string(int status);

/* ---- routing -----------------------------------------------------------
 * moe_route: GroupedTopK routing of [GTK] 三 3.1-3.6; plain top-k routing
 * ([MSG] 路由, select_experts) is the case num_expert_group = topk_group = 1.
 * Per token t:
 *   1. scores s = softmax over the row ([GTK] 3.1, max subtracted) or
 *      sigmoid of each logit (scoring = MOE_SCORING_SIGMOID);
 *   2. group score = MAX score inside each of the num_expert_group
 *      contiguous groups of E / num_expert_group experts ([GTK] 3.2);
 *   3. keep the topk_group best groups ([GTK] 3.3), mask the rest ([GTK] 3.4);
 *   4. topk best experts among the kept groups ([GTK] 3.5);
 *   5. if renormalize, divide the topk scores by their sum ([GTK] 3.6);
 *   6. multiply by routed_scaling_factor (always, last; [GTK] 3.6).
 * Ties (equal logits / equal group maxima) go to the lower index.  Outputs
 * are ordered by descending score.  Selection compares logits directly
 * (both scorings are monotone, [GTK] 七), so it does not depend on how the
 * scores round.  hidden_states play no part ([GTK] 二) and are not taken.
 *
 *   gating          [T, E] float32 router logits, row-major (read only).
 *   topk_weights    [T, topk] float32 out.
 *   topk_ids        [T, topk] int32 out, expert ids in [0, E).
 * Errors: NULL pointers (T > 0); T < 0; E < 1 or E > MOE_MAX_EXPERTS;
 * E % num_expert_group != 0; num_expert_group > 64; topk_group outside
 * [1, num_expert_group]; topk outside [1, MOE_MAX_TOPK] or larger than
 * topk_group * (E / num_expert_group) -> MOE_ERR_SHAPE / MOE_ERR_CONFIG.
 * NaN and +inf logits are outside the contract (no fault, unspecified ids);
 * -inf logits are allowed and rank last.  T = 0 is a no-op.
 */
MOE_API int moe_route(const float* gating, int64_t T, int32_t E, int32_t topk,
              int32_t num_expert_group, int32_t topk_group, int32_t scoring,
              int32_t renormalize, float routed_scaling_factor,
              float* topk_weights, int32_t* topk_ids, void* stream);

/* ---- alignment ---------------------------------------------------------
 * moe_align_block_size: [MSG] fused MoE, moe_align_block_size.  The pairs
 * are the num_pairs entries of the flattened topk_ids (pair i = token
 * i / topk, slot i % topk).  Pairs are grouped by expert in ascending expert
 * order, keeping ascending pair order inside each expert (a stable sort);
 * each expert's segment is padded with the placeholder value num_pairs up to
 * a multiple of block_m; experts without pairs get no segment.
 *
 *   topk_ids               [num_pairs] int32 in [0, E) (read only).
 *   sorted_token_ids       [max_padded] int32 out.  Entries [0, total) hold
 *                          the segments; entries [total, max_padded) are set
 *                          to num_pairs.
 *   expert_ids             [max_padded / block_m] int32 out: the expert of
 *                          each block of block_m entries; blocks at or past
 *                          total / block_m are set to -1 (an extension: the
 *                          GEMMs stop there without reading the total).
 *   num_tokens_post_padded [1] int32 out: total (a multiple of block_m).
 *   max_padded             capacity of sorted_token_ids; must be at least
 *                          moe_align_max_padded(num_pairs, E, block_m).
 *   ws, ws_bytes           optional device workspace of at least
 *                          moe_align_workspace_size(num_pairs, E) bytes
 *                          (16-byte aligned): with it the alignment runs as
 *                          two kernels (per-chunk counts, then placement);
 *                          NULL runs one kernel with no workspace.  Both give
 *                          identical outputs.
 * Null pointers are accepted only for buffers of capacity 0 (and topk_ids
 * when num_pairs = 0); num_tokens_post_padded is always written.
 * Errors: NULLs, num_pairs < 0 or >= 2^31, E outside [1, MOE_MAX_EXPERTS],
 * block_m outside [1, 1024], max_padded too small, workspace too small
 * (MOE_ERR_WORKSPACE).  Expert ids outside
 * [0, E) are outside the contract (they are dropped, not written).
 */
MOE_API int64_t moe_align_max_padded(int64_t num_pairs, int32_t E, int32_t block_m);

MOE_API size_t moe_align_workspace_size(int64_t num_pairs, int32_t E);

MOE_API int moe_align_block_size(const int32_t* topk_ids, int64_t num_pairs, int32_t E,
                         int32_t block_m, int32_t* sorted_token_ids,
                         int32_t* expert_ids, int32_t* num_tokens_post_padded,
                         int64_t max_padded, void* ws, size_t ws_bytes, void* stream);

/* ---- packed expert weights --------------------------------------------
 * moe_pack_weights: one-time re-layout of expert weights [E, N, K] (bf16 for
 * the MoE GEMMs, int8 for gmm_int8) for the MFMA tile kernels (block_m 64,
 * 128, 256 and the int8 GMM).  The weights and every result computed from
 * them are unchanged; only the byte order differs.  In the plain layout each
 * K step of a tile reads 64 bytes from each of 256 rows that lie K * element
 * size bytes apart; packed, the same step is one contiguous 16 KiB block,
 * which HBM serves far faster.
 *
 * Layout.  Each expert's rows are cut into tiles of 256 rows:
 *   epilogue MOE_EPILOGUE_NONE:     tile t holds rows 256t .. 256t+255;
 *   epilogue MOE_EPILOGUE_SILU_MUL: tile t holds gate rows 128t .. 128t+127
 *                                   and then the up rows N/2 + 128t ..
 *                                   (the pairs the SiLU*up epilogue joins).
 * K is cut into stages of 64 bytes (32 bf16 or 64 int8 elements).  Block
 * (e, t, s) is 16 KiB at byte offset ((e * NT + t) * KS + s) * 16384 with NT
 * tiles per expert and KS = ceil(K * element size / 64).  Inside a block, the
 * 16-byte chunk c (bytes 16c .. 16c+15 of the stage) of tile row r is at
 * r * 64 + 16 * (c ^ ((r >> 2) & 3)).  Rows past the matrix and bytes past K
 * are zero.
 *
 *   w         [E, N, K] of dtype (read only).
 *   dtype     MOE_DTYPE_BF16 or MOE_DTYPE_I8.
 *   epilogue  the epilogue of the GEMM that will use the packed weights.
 *   packed    output, at least moe_packed_weights_size(...) bytes.
 * Requirements: bf16 as moe_grouped_gemm for N and K; int8 as gmm_int8;
 * w and packed 16-byte aligned.  Errors: NULLs, bad sizes, dtype or
 * epilogue, packed_bytes too small.
 */
MOE_API size_t moe_packed_weights_size(int32_t dtype, int32_t E, int64_t N, int64_t K,
                                       int32_t epilogue);

MOE_API int moe_pack_weights(const void* w, int32_t dtype, int32_t E, int64_t N, int64_t K,
                     int32_t epilogue, void* packed, size_t packed_bytes, void* stream);

/* ---- grouped GEMM ------------------------------------------------------
 * moe_grouped_gemm: [MSG] fused MoE, fused_moe_kernel, with the gathered
 * weight never materialised ([P1] 01): for every block b of block_m entries
 * of sorted_token_ids below the device total, expert e = expert_ids[b], and
 * every entry p (pair index) < num_valid_pairs at sorted position s:
 *     a   = A row  (p / a_row_div  if a_rows == MOE_ROWS_PAIR,
 *                   s             if a_rows == MOE_ROWS_SORTED)
 *     acc = a . B[e]^T                       (fp32 accumulation, bf16 MFMA)
 *     EPILOGUE_NONE:     c = acc                               (N columns)
 *     EPILOGUE_SILU_MUL: c[j] = silu(acc[j]) * acc[N/2 + j]    (N/2 columns;
 *                        gate rows of B first, up rows second, [MSG] 练习 3)
 *     c *= topk_weights[p]                   (if topk_weights != NULL)
 *     C row (p if c_rows == MOE_ROWS_PAIR, s if MOE_ROWS_SORTED) = c.
 * Placeholder entries (p >= num_valid_pairs) are neither read nor written.
 *
 *   A        rows of K elements, row stride lda elements; a_dtype BF16 or
 *            F32 (F32 rows are rounded to bf16 on load).
 *   B        [E, N, K] bf16, K contiguous (b_layout MOE_WEIGHTS_PLAIN), or
 *            written by moe_pack_weights with the same E, N, K and epilogue
 *            (MOE_WEIGHTS_PACKED; block_m 64, 128 or 256 and bf16 A only).
 *   C        row stride ldc elements; c_dtype F32, BF16 or F16.
 *   sorted_token_ids / expert_ids / num_tokens_post_padded: as written by
 *            moe_align_block_size with the same block_m; max_padded is the
 *            capacity of sorted_token_ids (the launch is sized by it and the
 *            device total cuts it short).
 *   block_m  16 or 32 (weight-streaming kernel for few rows per expert) or
 *            64, 128 or 256 (MFMA tile kernel; 256 needs bf16 A).
 * Requirements: K % 8 == 0, N % 16 == 0 (SILU_MUL: (N/2) % 16 == 0),
 * lda >= K and ldc >= output width, both multiples of 8; A, B and C
 * 16-byte aligned.
 */
MOE_API int moe_grouped_gemm(const void* A, int32_t a_dtype, int64_t lda, int32_t a_rows,
                     int32_t a_row_div, const void* B, int32_t b_layout, int32_t E, int64_t N,
                     int64_t K, const int32_t* sorted_token_ids,
                     const int32_t* expert_ids,
                     const int32_t* num_tokens_post_padded, int64_t max_padded,
                     int32_t block_m, int64_t num_valid_pairs,
                     const float* topk_weights, int32_t epilogue, void* C,
                     int32_t c_dtype, int64_t ldc, int32_t c_rows, void* stream);

/* ---- grouped GEMM on expert-wide tiles ----------------------------------
 * The same GEMM as moe_grouped_gemm at block_m 32, with its work cut into
 * tiles of up to 10 consecutive blocks (320 sorted entries) of one expert
 * times 256 rows of B, so each slice of an expert's weights is read by one
 * tile (by two or more only for experts of more than 320 entries).  The
 * MFMA sequence over K is the tile kernels' one: C is bit-identical to
 * moe_grouped_gemm at block_m 64 or 128 for the same rows.  Scheduling
 * follows [GMM] 3.3 and 4.1: work is assigned per expert, with large
 * experts cut into tiles of near-equal size so that no tile holds much more
 * than another; a workgroup takes one tile (160 KiB of LDS, one per CU).
 *
 * moe_wide_tile_table_size: ints of the tile table for a block-32
 *   alignment of capacity max_padded (-1 if max_padded is negative or not a
 *   multiple of 32).
 * moe_wide_tile_table: writes the table from moe_align_block_size's output
 *   at block_m 32: table[0] = number of tiles; tile j: table[1 + 3j] =
 *   expert, table[2 + 3j] = first block, table[3 + 3j] = blocks (1..10); an
 *   expert of n blocks gets ceil(n / 10) tiles of near-equal size.  One
 *   launch; E <= 1024 (MOE_ERR_CONFIG otherwise); table_ints below the size
 *   above is MOE_ERR_WORKSPACE.
 * moe_grouped_gemm_wide: moe_grouped_gemm's arguments with tile_table (as
 *   written by moe_wide_tile_table for the same alignment) in place of
 *   block_m.  A and C bf16 only (MOE_ERR_DTYPE otherwise); SILU_MUL takes no
 *   topk_weights (MOE_ERR_CONFIG); plain or packed B; E <= 1024.  Table
 *   entries outside the alignment's blocks or experts are skipped.  Needs
 *   160 KiB of LDS per workgroup (one per CU).
 */
MOE_API int64_t moe_wide_tile_table_size(int64_t max_padded);
MOE_API int moe_wide_tile_table(const int32_t* expert_ids, const int32_t* num_tokens_post_padded,
                                int32_t E, int64_t max_padded, int32_t* table,
                                int64_t table_ints, void* stream);
MOE_API int moe_grouped_gemm_wide(const void* A, int32_t a_dtype, int64_t lda, int32_t a_rows,
                                  int32_t a_row_div, const void* B, int32_t b_layout, int32_t E,
                                  int64_t N, int64_t K, const int32_t* sorted_token_ids,
                                  const int32_t* expert_ids,
                                  const int32_t* num_tokens_post_padded, int64_t max_padded,
                                  const int32_t* tile_table, int64_t num_valid_pairs,
                                  const float* topk_weights, int32_t epilogue, void* C,
                                  int32_t c_dtype, int64_t ldc, int32_t c_rows, void* stream);

/* ---- whole layer -------------------------------------------------------
 * moe_forward: [MSG] fused MoE, FusedMoeBackend.forward, with routing per
 * moe_route: route -> align -> gate_up GEMM with silu(gate)*up in its
 * epilogue (intermediate h kept in sorted order, bf16) -> down GEMM times
 * the routing weight -> per-token sum over the topk slots, written in x's
 * dtype.  out[t] = sum_k w[t,k] * W2[e] (silu(W1g[e] x[t]) * (W1u[e] x[t])).
 * The GEMMs are two launches (gate_up into h in sorted order, then down
 * into per-pair rows y) and the sum is a third.  At block_m 32 with bf16 x
 * (and E <= 1024) they run on expert-wide tiles: a small launch builds a
 * table of tiles of up to 320 consecutive rows of one expert, and each tile
 * multiplies them against 256 weight rows, so every weight slice is read
 * once per expert; results are bit-identical to the moe_grouped_gemm tile
 * kernels (same MFMA sequence over K).  Otherwise the GEMMs are two
 * moe_grouped_gemm launches.
 *
 *   x        [T, H] bf16 or f32 (x_dtype); out [T, H] in the same dtype.
 *   gating   [T, E] f32 logits.
 *   w1       [E, 2I, H] bf16 (gate rows [0, I), up rows [I, 2I)).
 *   w2       [E, H, I] bf16.
 *   w_layout MOE_WEIGHTS_PLAIN, or MOE_WEIGHTS_PACKED: w1 packed with
 *            MOE_EPILOGUE_SILU_MUL and w2 with MOE_EPILOGUE_NONE by
 *            moe_pack_weights (needs bf16 x; block_m 32, 64, 128 or 256).
 *   topk_weights_out [T, topk] f32, topk_ids_out [T, topk] int32: optional
 *            (NULL = kept in the workspace only).
 *   block_m  0 = chosen from the average pairs per expert (with bf16 x: 32,
 *            the expert-wide tiles, at 96 or more pairs per expert and
 *            E <= 1024, else 64 or 128;
 *            16, 32, 64 or 128 for f32 x on plain weights); otherwise one of
 *            the moe_grouped_gemm block sizes.  With 0, plain weights and a
 *            small layer (T * topk <= 2048 and 6 * T * topk * H * I <= 2^28)
 *            the alignment and the tiled GEMMs are skipped: after routing
 *            one launch computes each token's pairs in k order in fp32 (x
 *            as given, h in fp32) and writes out.
 *   ws       device workspace of at least moe_forward_workspace_size(...)
 *            bytes for the same arguments (256-byte aligned).
 * Requirements: H % 16 == 0, I % 16 == 0, plus moe_route's.
 */
/* Block size moe_forward uses when called with block_m = 0 (the choice is a
 * pure function of the shape, x's dtype and the weight layout); -1 on
 * invalid arguments. */
MOE_API int32_t moe_forward_block_m(int64_t T, int32_t E, int32_t topk, int32_t x_dtype,
                                    int32_t w_layout);

MOE_API size_t moe_forward_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E,
                                  int32_t topk, int32_t block_m);

MOE_API int moe_forward(const void* x, int32_t x_dtype, const float* gating,
                const void* w1, const void* w2, int32_t w_layout, int64_t T, int32_t H, int32_t I,
                int32_t E, int32_t topk, int32_t num_expert_group,
                int32_t topk_group, int32_t scoring, int32_t renormalize,
                float routed_scaling_factor, int32_t block_m, void* out,
                float* topk_weights_out, int32_t* topk_ids_out, void* ws,
                size_t ws_bytes, void* stream);

/* moe_forward_noalloc: moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as moe_forward,
 * without ws / ws_bytes: the workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES per device, part of the library's code object,
 * held from the library's first use on a device until the process ends.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * call) and runs the same kernels as moe_forward.
 *   MOE_ERR_WORKSPACE  the layer needs more than MOE_NOALLOC_SCRATCH_BYTES
 *                      (moe_forward_workspace_size gives the need; 96 MiB
 *                      covers, e.g., T = 64 tokens at H = 7168, I = 2048,
 *                      E = 256, top-8);
 *   MOE_ERR_HIP        the scratch address could not be obtained.
 * Every call on a device shares that device's one array and leaves its
 * contents behind: calls that overlap on one device (other streams, other
 * host threads) race and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
MOE_API int moe_forward_noalloc(const void* x, int32_t x_dtype, const float* gating,
                const void* w1, const void* w2, int32_t w_layout, int64_t T, int32_t H, int32_t I,
                int32_t E, int32_t topk, int32_t num_expert_group,
                int32_t topk_group, int32_t scoring, int32_t renormalize,
                float routed_scaling_factor, int32_t block_m, void* out,
                float* topk_weights_out, int32_t* topk_ids_out, void* stream);

/* ---- INT8 activations and the INT8 fused layer ------------------------
 * moe_quantize_rows: symmetric per-row int8 quantisation, [GMM] 3.2 (per
 * token for activations): scale[r] = max|x[r, :]| / 127 (1 for an all-zero
 * row), q[r, c] = clamp(round_half_even(x[r, c] / scale[r]), -127, 127).
 * Computed in float32 with IEEE division, so the codes are a pure function
 * of the row's float32 values.
 *   x       [rows, ld] f32 or bf16 (x_dtype), first cols used.
 *   q       [rows, cols] int8 out.      scales  [rows] f32 out.
 * Requirements: cols % 8 == 0, ld >= cols, ld % 8 == 0, x and q 16-byte
 * aligned.  rows = 0 is a no-op.
 */
MOE_API int moe_quantize_rows(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                              int64_t ld, int8_t* q, float* scales, void* stream);

/* moe_forward_w8a8: moe_forward with int8 weights and int8 activations in
 * both GEMMs (per-channel weight scales and per-token activation scales,
 * [GMM] 3.2; exact int32 sums, [GMM] 5.3; activations quantised before
 * their GEMM, [GMM] 4):
 *   xq, sx = moe_quantize_rows(x)
 *   h[pair] = silu(gate) * up, gate/up[n] = sx[t] * w1_scales[e, n] *
 *             sum_k xq[t, k] * w1q[e, n, k]      (float32, stored as bf16)
 *   hq, sh = per-row int8 of the bf16 h (one row per pair)
 *   out[t] = sum_k w[t,k] * sh[pair] * w2_scales[e, n] * sum_j hq[j] * w2q[e, n, j]
 * Routing, alignment and the final reduce are moe_forward's.
 *   w1q [E, 2I, H] int8 and w1_scales [E, 2I] f32; w2q [E, H, I] int8 and
 *   w2_scales [E, H] f32; with w_layout MOE_WEIGHTS_PACKED, w1q packed by
 *   moe_pack_weights(MOE_DTYPE_I8, MOE_EPILOGUE_SILU_MUL) and w2q with
 *   MOE_EPILOGUE_NONE.
 *   x [T, H] bf16 or f32; out [T, H] in x's dtype.
 *   block_m  0 (chosen: 32, the expert-wide int8 tiles, for bf16 x at 96 or
 *            more pairs per expert and E <= 1024, else at least 64), 32
 *            (bf16 x only), 64, 128 or 256.  The expert-wide tiles give the
 *            same bits as the 256 x 128 / 256 x 64 tiles (exact int32 sums).
 *   ws       at least moe_forward_w8a8_workspace_size(...) bytes, 256-byte
 *            aligned.
 * Requirements: H % 16 == 0, I % 16 == 0, H and I <= 131072, plus
 * moe_route's; scale arrays 16-byte aligned.
 */
MOE_API size_t moe_forward_w8a8_workspace_size(int64_t T, int32_t H, int32_t I, int32_t E,
                                               int32_t topk, int32_t block_m);

MOE_API int moe_forward_w8a8(const void* x, int32_t x_dtype, const float* gating,
                             const int8_t* w1q, const float* w1_scales, const int8_t* w2q,
                             const float* w2_scales, int32_t w_layout, int64_t T, int32_t H,
                             int32_t I, int32_t E, int32_t topk, int32_t num_expert_group,
                             int32_t topk_group, int32_t scoring, int32_t renormalize,
                             float routed_scaling_factor, int32_t block_m, void* out,
                             float* topk_weights_out, int32_t* topk_ids_out, void* ws,
                             size_t ws_bytes, void* stream);

/* ---- INT8 grouped GEMM -------------------------------------------------
 * gmm_int8: [GMM] 2.1 and 3.1.  The input rows are sorted by expert; rows
 * [expert_offsets[e], expert_offsets[e+1]) belong to expert e, and
 *   output[m, n] = fp16( scales_x[m] * scales_w[e, n] *
 *                        sum_k input[m, k] * weights[e, n, k] )
 * with the integer sum accumulated exactly in int32 ([GMM] 5.3) and the
 * scales applied in fp32.  Output rows stay in input order.
 *
 *   input          [M, K] int8.       weights   [E, N, K] int8 (K contiguous);
 *                  with w_layout MOE_WEIGHTS_PACKED, written by
 *                  moe_pack_weights(dtype MOE_DTYPE_I8, epilogue NONE).
 *   scales_x       [M] f32 per row.   scales_w  [E, N] f32 per output channel.
 *   expert_offsets [E + 1] int32, non-decreasing, offsets[0] = 0,
 *                  offsets[E] = M (device memory; checked on the device only
 *                  by clamping, so rows outside [0, M) are never touched).
 *   expert_sizes   optional [E] int32 (may be NULL); the offsets decide.
 *   output         [M, N] fp16.
 * Requirements: K % 16 == 0, N % 16 == 0, K <= 131072 (exact int32 sums),
 * E in [1, MOE_MAX_EXPERTS].
 */
MOE_API int gmm_int8(const int8_t* input, const int8_t* weights, int32_t w_layout, const float* scales_x,
             const float* scales_w, const int32_t* expert_offsets,
             const int32_t* expert_sizes, void* output, int64_t M, int64_t K,
             int64_t N, int32_t E, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

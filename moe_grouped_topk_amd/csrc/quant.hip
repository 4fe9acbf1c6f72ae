// Per-row symmetric int8 quantisation (low-precision GMM article, section
// 3.2: scale = max|row| / 127, codes rounded half to even and clamped to
// +-127), taken in float32 with IEEE division so that codes are a pure
// function of the row's float32 values.  Feeds the int8 GEMMs: activations
// per token, the intermediate h per pair row.
//
// Rows of up to 2048 columns stay in registers between the row's max |x| and
// its codes (one read of the row): 32 or 64 lanes per row, up to 4 chunks of
// 8 values per lane (16-byte bf16 loads, 8-byte stores), two rows per wave
// when 32 lanes hold the row.  Longer rows: one wave per row, read twice.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kQuantWaves = 4;

// cols % 8 == 0; rows 16-byte aligned (checked by the callers).  One wave
// per row of any length: the row is read once for its maximum and once for
// its codes.
template <int XDT>
__global__ void __launch_bounds__(kQuantWaves * kWave)
quantize_rows_kernel(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                     const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ total,
                     int64_t num_valid, int8_t* __restrict__ q, float* __restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r = (int64_t)blockIdx.x * kQuantWaves + threadIdx.x / kWave;
  if (r >= rows) return;
  if (sorted_ids) {
    if (r >= *total) return;
    const int p = sorted_ids[r];
    if (p < 0 || p >= num_valid) return;
  }
  constexpr int eb = XDT == 1 ? 2 : 4;
  const void* row = reinterpret_cast<const uint8_t*>(x) + r * ld * eb;
  int8_t* qrow = q + r * cols;
  float amax = 0.0f;
  for (int64_t i = (int64_t)lane * 8; i < cols; i += kWave * 8) {
    float v[8];
    load8<XDT>(row, i, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  const float scale = quant_scale(amax);
  for (int64_t i = (int64_t)lane * 8; i < cols; i += kWave * 8) {
    float v[8];
    load8<XDT>(row, i, v);
    *reinterpret_cast<uint2*>(qrow + i) = make_uint2(code4(v, scale), code4(v + 4, scale));
  }
  if (lane == 0) scales[r] = scale;
}

// Rows of at most CH * LPR * 8 columns: LPR lanes per row (64 / LPR rows per
// wave), CH chunks of 8 values per lane, the maximum over the row's lanes.
template <int XDT, int CH, int LPR>
__global__ void __launch_bounds__(kQuantWaves * kWave)
quantize_rows_reg_kernel(const void* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                         const int32_t* __restrict__ sorted_ids, const int32_t* __restrict__ total,
                         int64_t num_valid, int8_t* __restrict__ q, float* __restrict__ scales) {
  static_assert(kWave % LPR == 0 && CH >= 1, "lanes per row");
  constexpr int RPW = kWave / LPR;
  const int lane = threadIdx.x & (kWave - 1), l = lane % LPR;
  const int64_t r = ((int64_t)blockIdx.x * kQuantWaves + threadIdx.x / kWave) * RPW + lane / LPR;
  const bool in = r < rows;
  // the row's values are loaded alongside its pair id, not after it (a
  // row of the padded range is readable whether or not it holds a pair)
  constexpr int eb = XDT == 1 ? 2 : 4;
  const void* row = reinterpret_cast<const uint8_t*>(x) + (in ? r : 0) * ld * eb;
  float v[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t i = ((int64_t)c * LPR + l) * 8;
    if (in && i < cols) load8<XDT>(row, i, v[c]);
  }
  bool live = in;
  if (in && sorted_ids) {
    const int p = sorted_ids[r];
    live = r < *total && p >= 0 && p < num_valid;
  }
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t i = ((int64_t)c * LPR + l) * 8;
    if (live && i < cols) {
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[c][k]));
    }
  }
  // every lane takes part (the row groups are aligned runs of LPR lanes)
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  if (!live) return;
  const float scale = quant_scale(amax);
  int8_t* qrow = q + r * cols;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t i = ((int64_t)c * LPR + l) * 8;
    if (i < cols)
      *reinterpret_cast<uint2*>(qrow + i) = make_uint2(code4(v[c], scale), code4(v[c] + 4, scale));
  }
  if (l == 0) scales[r] = scale;
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld,
                                const int32_t* sorted_ids, const int32_t* total, int64_t num_valid,
                                int8_t* q, float* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 block(kQuantWaves * kWave);
  const int64_t chunks = cols / 8;                  // 8-value chunks of a row
  auto reg = [&](auto k, int rpw) {
    const dim3 grid((unsigned)((rows + kQuantWaves * rpw - 1) / (kQuantWaves * rpw)));
    hipLaunchKernelGGL(k, grid, block, 0, stream, x, rows, cols, ld, sorted_ids, total, num_valid,
                       q, scales);
  };
#define MOE_QUANT_REG(XDT)                                                                     \
  if (chunks <= 32) reg(quantize_rows_reg_kernel<XDT, 1, 32>, 2);                             \
  else if (chunks <= 64) reg(quantize_rows_reg_kernel<XDT, 2, 32>, 2);                        \
  else if (chunks <= 96) reg(quantize_rows_reg_kernel<XDT, 3, 32>, 2);                        \
  else if (chunks <= 128) reg(quantize_rows_reg_kernel<XDT, 2, 64>, 1);                       \
  else if (chunks <= 192) reg(quantize_rows_reg_kernel<XDT, 3, 64>, 1);                       \
  else if (chunks <= 256) reg(quantize_rows_reg_kernel<XDT, 4, 64>, 1);                       \
  else hipLaunchKernelGGL((quantize_rows_kernel<XDT>),                                      \
                          dim3((unsigned)((rows + kQuantWaves - 1) / kQuantWaves)), block, 0,  \
                          stream, x, rows, cols, ld, sorted_ids, total, num_valid, q, scales)
  if (x_dtype == 1) {
    MOE_QUANT_REG(1);
  } else {
    MOE_QUANT_REG(0);
  }
#undef MOE_QUANT_REG
  return hipGetLastError();
}

}  // namespace moe

// Per-row symmetric int8 quantisation (low-precision GMM article, section
// 3.2: scale = max|row| / 127, codes rounded half to even and clamped to
// +-127), taken in float32 with IEEE division so that codes are a pure
// function of the row's float32 values.  Feeds the int8 GEMMs: activations
// per token, the intermediate h per pair row.
//
// One wave per row: the row's max |x| by a wave max, then the codes, 8
// elements per lane per step (16-byte bf16 loads, 8-byte stores); rows up to
// 2048 columns stay in registers between the two.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kQuantWaves = 4;

// cols % 8 == 0; rows 16-byte aligned (checked by the callers).
//   CH > 0: rows of at most CH * 512 columns, held in registers (CH chunks of
//   8 values per lane): one read of the row.  CH = 0: any length, the row is
//   read once for its maximum and once for its codes.
template <int XDT, int CH>
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
  if constexpr (CH > 0) {
    float v[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t i = ((int64_t)c * kWave + lane) * 8;
      if (i < cols) {
        load8<XDT>(row, i, v[c]);
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[c][k]));
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    const float scale = quant_scale(amax);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t i = ((int64_t)c * kWave + lane) * 8;
      if (i < cols)
        *reinterpret_cast<uint2*>(qrow + i) = make_uint2(code4(v[c], scale), code4(v[c] + 4, scale));
    }
    if (lane == 0) scales[r] = scale;
  } else {
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
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld,
                                const int32_t* sorted_ids, const int32_t* total, int64_t num_valid,
                                int8_t* q, float* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + kQuantWaves - 1) / kQuantWaves));
  const dim3 block(kQuantWaves * kWave);
#define MOE_QUANT(XDT, CH)                                                                     \
  hipLaunchKernelGGL((quantize_rows_kernel<XDT, CH>), grid, block, 0, stream, x, rows, cols, ld, \
                     sorted_ids, total, num_valid, q, scales)
  const int64_t chunks = (cols / 8 + kWave - 1) / kWave;   // 8-value chunks per lane
  if (x_dtype == 1) {
    if (chunks <= 2) MOE_QUANT(1, 2);
    else if (chunks <= 4) MOE_QUANT(1, 4);
    else MOE_QUANT(1, 0);
  } else {
    if (chunks <= 2) MOE_QUANT(0, 2);
    else if (chunks <= 4) MOE_QUANT(0, 4);
    else MOE_QUANT(0, 0);
  }
#undef MOE_QUANT
  return hipGetLastError();
}

}  // namespace moe

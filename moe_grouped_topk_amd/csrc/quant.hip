// Per-row symmetric int8 quantisation (low-precision GMM article, section
// 3.2: scale = max|row| / 127, codes rounded half to even and clamped to
// +-127), taken in float32 with IEEE division so that codes are a pure
// function of the row's float32 values.  Feeds the int8 GEMMs: activations
// per token, the intermediate h per pair row.
//
// One wave per row.  Pass 1: the row's max |x| by a wave max; pass 2: the
// codes, 8 elements per lane per step (16-byte bf16 loads, 8-byte stores).

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kQuantWaves = 4;

template <int XDT>
__device__ __forceinline__ void load8(const void* row, int64_t i, float (&v)[8]) {
  if constexpr (XDT == 1) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(row) + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(u[k] << 16);
      v[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  } else {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(row) + i);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(row) + i + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[4 + k] = b[k];
    }
  }
}

__device__ __forceinline__ uint32_t code4(const float* v, float scale) {
  uint32_t r = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float q = rintf(v[k] / scale);               // IEEE division, round half to even
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    r |= ((uint32_t)(int32_t)q & 0xffu) << (8 * k);
  }
  return r;
}

// cols % 8 == 0; rows 16-byte aligned (checked by the callers).
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
  float amax = 0.0f;
  for (int64_t i = (int64_t)lane * 8; i < cols; i += kWave * 8) {
    float v[8];
    load8<XDT>(row, i, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
  const float scale = amax == 0.0f ? 1.0f : amax / 127.0f;
  int8_t* qrow = q + r * cols;
  for (int64_t i = (int64_t)lane * 8; i < cols; i += kWave * 8) {
    float v[8];
    load8<XDT>(row, i, v);
    *reinterpret_cast<uint2*>(qrow + i) = make_uint2(code4(v, scale), code4(v + 4, scale));
  }
  if (lane == 0) scales[r] = scale;
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld,
                                const int32_t* sorted_ids, const int32_t* total, int64_t num_valid,
                                int8_t* q, float* scales, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + kQuantWaves - 1) / kQuantWaves));
  if (x_dtype == 1)
    hipLaunchKernelGGL(quantize_rows_kernel<1>, grid, dim3(kQuantWaves * kWave), 0, stream, x, rows,
                       cols, ld, sorted_ids, total, num_valid, q, scales);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<0>, grid, dim3(kQuantWaves * kWave), 0, stream, x, rows,
                       cols, ld, sorted_ids, total, num_valid, q, scales);
  return hipGetLastError();
}

}  // namespace moe

// Device-side helpers shared by the gfx950 kernels of the fused-MoE path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr int kWave = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies, 32 CUs each

// Order-preserving 32-bit key of a float: a > b  <=>  key(a) > key(b) for
// non-NaN values; -0.0 is folded onto +0.0 so equal values get equal keys.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of float_key (exact).
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = __shfl_xor((uint32_t)v, mask, kWave);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), mask, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp each);
// for z -> -inf the reciprocal of +inf gives 0, for z -> +inf it gives z.
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Two floats -> two bfloat16 (a in the low half), round to nearest even,
// NaN kept a NaN.  One gfx950 packed conversion (v_cvt_pk_bf16_f32) in place
// of the integer rounding sequence per value.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const f32x2_v v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// Store 4 consecutive fp32 values converted to the output dtype
// (0 = f32, 1 = bf16, 2 = f16).  dst is element-aligned to 4 elements.
template <int CDT>
__device__ __forceinline__ void store4(void* dst, float a, float b, float c, float d) {
  if constexpr (CDT == 0) {
    f32x4_t v = {a, b, c, d};
    *reinterpret_cast<f32x4_t*>(dst) = v;
  } else if constexpr (CDT == 1) {
    uint2 v = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
    *reinterpret_cast<uint2*>(dst) = v;
  } else {
    uint2 v = make_uint2(pack_f16x2(a, b), pack_f16x2(c, d));
    *reinterpret_cast<uint2*>(dst) = v;
  }
}

// Per-row symmetric int8 quantisation (low-precision GMM article, section
// 3.2): scale = max|row| / 127 (1 for an all-zero row), codes
// round-half-to-even(x / scale) clamped to +-127, in float32 with IEEE
// division, so the codes are a pure function of the row's float32 values
// whichever kernel computes them.
//   load8: eight consecutive row values (XDT 1: bf16, 16-byte load;
//   0: f32, two 16-byte loads) as float32.
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

__device__ __forceinline__ float quant_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / 127.0f;
}

// Four codes packed little-endian into 32 bits.
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

template <int CDT> struct ElemBytes;
template <> struct ElemBytes<0> { static constexpr int value = 4; };
template <> struct ElemBytes<1> { static constexpr int value = 2; };
template <> struct ElemBytes<2> { static constexpr int value = 2; };

}  // namespace moe

// Weight-streaming grouped GEMM for few rows per expert (block_m 16 or 32).
//
// Semantics: identical to the tile kernel (mini-sglang "MoE and fused MoE",
// fused_moe_kernel, with the SiLU(gate)*up epilogue of its exercise 3); the
// page's exercise 1 answer notes that at decode sizes a 64-row block is
// almost all padding and asks for small blocks or per-expert GEMV.
//
// gfx950 design: at a few tokens per expert the layer only has to read each
// touched expert's weights once at HBM rate; MFMA waste does not matter.  The
// weights take the 16-row slot of v_mfma_f32_16x16x32_bf16 and the block's
// tokens its 16-column slot (the role the swap-AB trick of the spke.com
// article gives the large dimension on Hopper).  One wave64 streams 32 weight
// rows (gate+up rows of 16 intermediate columns, or 32 output rows) over the
// whole of K; no LDS is used.  Per 256-element K chunk, lane l reads 128
// contiguous bytes of weight row (l & 15) at byte offset 128*(l >> 4) and the
// same K range of token (l & 15); the 8 MFMA steps of the chunk each take
// 16 of those bytes.  Any assignment of K indices to (lane group, step) is
// valid as long as both operands use the same one, which they do.  Two
// register buffers keep the next chunk's loads in flight during the MFMAs.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kChunkBytes = 512;    // bf16 bytes of K per chunk (256 elements)
constexpr int kMaxTopkUnroll = 8;   // y rows loaded together by the reduce

template <int TG, bool TF32>
struct Regs {
  u32x4_t w[2][8];
  u32x4_t t[TG][TF32 ? 16 : 8];
};

template <int TG, int EPI, bool TF32, int CDT>
__global__ void __launch_bounds__(kThreads) moe_gemm_stream_kernel(MoeGemmArgs a) {
  constexpr int BMS = TG * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int nslice = EPI ? (int)((Nout + 63) / 64) : (int)((a.N + 127) / 128);
  const int blk = (int)blockIdx.x / nslice, sl = (int)blockIdx.x % nslice;
  const int nblk = *a.total / BMS;
  if (blk >= nblk) return;
  const int e = a.expert_ids[blk];
  if (e < 0) return;
  const int64_t s0 = (int64_t)blk * BMS;

  // Tokens of this block: lane (l & 15) of group cb.
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(a.A);
  const int64_t a_row_bytes = a.lda * (TF32 ? 4 : 2);
  int pair[TG];
  const uint8_t* tp[TG];
  uint32_t active = 0u;
#pragma unroll
  for (int cb = 0; cb < TG; ++cb) {
    const int64_t s = s0 + cb * 16 + (lane & 15);
    const int p = a.sorted_ids[s];
    const bool ok = p >= 0 && p < a.num_valid;
    pair[cb] = ok ? p : -1;
    const int64_t src = (a.a_rows == 0) ? (int64_t)(p / a.a_row_div) : s;
    tp[cb] = ok ? Ab + src * a_row_bytes : nullptr;
    if (__ballot(ok) != 0ull) active |= 1u << cb;
  }

  // Weight rows of this wave: two 16-row blocks.
  const uint8_t* Bw = reinterpret_cast<const uint8_t*>(a.B);
  const int64_t kbytes = a.K * 2;
  const uint8_t* wp[2];
  int64_t col0;
  if (EPI) {
    const int64_t hcol = (int64_t)sl * 64 + wave * 16 + (lane & 15);
    const bool ok = hcol < Nout;
    wp[0] = ok ? Bw + ((int64_t)e * a.N + hcol) * kbytes : nullptr;
    wp[1] = ok ? Bw + ((int64_t)e * a.N + Nout + hcol) * kbytes : nullptr;
    col0 = (int64_t)sl * 64 + wave * 16;
  } else {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t n = (int64_t)sl * 128 + wave * 32 + rb * 16 + (lane & 15);
      wp[rb] = n < a.N ? Bw + ((int64_t)e * a.N + n) * kbytes : nullptr;
    }
    col0 = (int64_t)sl * 128 + wave * 32;
  }
  if (col0 >= Nout) return;   // whole wave past the last column (no barriers here)

  const int g = lane >> 4;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  auto load = [&](Regs<TG, TF32>& r, int c) {
    const int64_t base = (int64_t)c * kChunkBytes + g * 128;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int64_t off = base + s * 16;
        r.w[rb][s] = (wp[rb] && off < kbytes) ? *reinterpret_cast<const u32x4_t*>(wp[rb] + off) : zero;
      }
#pragma unroll
    for (int cb = 0; cb < TG; ++cb) {
      if (!((active >> cb) & 1u)) continue;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int64_t off = base + s * 16;
        const bool ok = tp[cb] && off < kbytes;
        if constexpr (TF32) {
          r.t[cb][2 * s] = ok ? *reinterpret_cast<const u32x4_t*>(tp[cb] + 2 * off) : zero;
          r.t[cb][2 * s + 1] = ok ? *reinterpret_cast<const u32x4_t*>(tp[cb] + 2 * off + 16) : zero;
        } else {
          r.t[cb][s] = ok ? *reinterpret_cast<const u32x4_t*>(tp[cb] + off) : zero;
        }
      }
    }
  };

  f32x4_t acc[2][TG];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int cb = 0; cb < TG; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Regs<TG, TF32>& r) {
#pragma unroll
    for (int cb = 0; cb < TG; ++cb) {
      if (!((active >> cb) & 1u)) continue;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        u32x4_t tv;
        if constexpr (TF32) {
          const u32x4_t lo = r.t[cb][2 * s], hi = r.t[cb][2 * s + 1];
          tv[0] = pack_bf16x2(__uint_as_float(lo[0]), __uint_as_float(lo[1]));
          tv[1] = pack_bf16x2(__uint_as_float(lo[2]), __uint_as_float(lo[3]));
          tv[2] = pack_bf16x2(__uint_as_float(hi[0]), __uint_as_float(hi[1]));
          tv[3] = pack_bf16x2(__uint_as_float(hi[2]), __uint_as_float(hi[3]));
        } else {
          tv = r.t[cb][s];
        }
        const bf16x8_t bt = __builtin_bit_cast(bf16x8_t, tv);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, r.w[rb][s]), bt, acc[rb][cb], 0, 0, 0);
      }
    }
  };

  const int nch = (int)((kbytes + kChunkBytes - 1) / kChunkBytes);
  Regs<TG, TF32> ra, rb_;
  load(ra, 0);
  for (int c = 0; c < nch; c += 2) {
    if (c + 1 < nch) load(rb_, c + 1);
    compute(ra);
    if (c + 1 < nch) {
      if (c + 2 < nch) load(ra, c + 2);
      compute(rb_);
    }
  }

  // Epilogue: lane holds features 4*(lane>>4) + [0,4) of each row block for
  // token (lane & 15) of each group.
  uint8_t* Cb = reinterpret_cast<uint8_t*>(a.C);
  constexpr int ce = ElemBytes<CDT>::value;
#pragma unroll
  for (int cb = 0; cb < TG; ++cb) {
    const int p = pair[cb];
    if (p < 0) continue;
    const int64_t s = s0 + cb * 16 + (lane & 15);
    const int64_t crow = (a.c_rows == 0) ? (int64_t)p : s;
    const float w = a.topk_weights ? a.topk_weights[p] : 1.0f;
    uint8_t* rowp = Cb + crow * a.ldc * ce;
    if (EPI) {
      const int64_t col = col0 + 4 * (lane >> 4);
      if (col < Nout) {
        const f32x4_t gt = acc[0][cb], up = acc[1][cb];
        store4<CDT>(rowp + col * ce, silu_f32(gt[0]) * up[0] * w, silu_f32(gt[1]) * up[1] * w,
                    silu_f32(gt[2]) * up[2] * w, silu_f32(gt[3]) * up[3] * w);
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int64_t col = col0 + rb * 16 + 4 * (lane >> 4);
        if (col < a.N) {
          const f32x4_t v = acc[rb][cb];
          store4<CDT>(rowp + col * ce, v[0] * w, v[1] * w, v[2] * w, v[3] * w);
        }
      }
    }
  }
}

template <int TG, int EPI, bool TF32, int CDT>
hipError_t launch_t(const MoeGemmArgs& a, hipStream_t stream) {
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int nslice = EPI ? (int)((Nout + 63) / 64) : (int)((a.N + 127) / 128);
  const int64_t grid = (a.max_padded / (TG * 16)) * nslice;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((moe_gemm_stream_kernel<TG, EPI, TF32, CDT>), dim3((unsigned)grid),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int TG, int EPI, bool TF32>
hipError_t launch_c(const MoeGemmArgs& a, hipStream_t s) {
  switch (a.c_dtype) {
    case 0: return launch_t<TG, EPI, TF32, 0>(a, s);
    case 1: return launch_t<TG, EPI, TF32, 1>(a, s);
    default: return launch_t<TG, EPI, TF32, 2>(a, s);
  }
}

template <int TG>
hipError_t launch_tg(const MoeGemmArgs& a, hipStream_t s) {
  const bool tf32 = a.a_dtype == 0;
  if (a.epilogue) return tf32 ? launch_c<TG, 1, true>(a, s) : launch_c<TG, 1, false>(a, s);
  return tf32 ? launch_c<TG, 0, true>(a, s) : launch_c<TG, 0, false>(a, s);
}

// out[t, :] = sum_k y[t * topk + k, :], summed in fp32 in the order
// k = 0 .. topk-1 (YDT: y is f32 (0) or bf16 (1)).
template <int YDT>
__device__ __forceinline__ f32x4_t load4(const uint8_t* p) {
  if constexpr (YDT == 0) {
    return *reinterpret_cast<const f32x4_t*>(p);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return f32x4_t{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                   __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
  }
}

template <int YDT, int CDT>
__global__ void __launch_bounds__(256) topk_reduce_kernel(const void* __restrict__ y, int64_t T,
                                                          int topk, int64_t H, void* out) {
  constexpr int ye = YDT == 0 ? 4 : 2;
  const int64_t q = H / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * q) return;
  const int64_t t = idx / q, c = (idx % q) * 4;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(y) + ((t * topk) * H + c) * ye;
  f32x4_t v[kMaxTopkUnroll];
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  int k = 0;
  for (; k + kMaxTopkUnroll <= topk; k += kMaxTopkUnroll) {
#pragma unroll
    for (int j = 0; j < kMaxTopkUnroll; ++j) v[j] = load4<YDT>(src + (int64_t)(k + j) * H * ye);
#pragma unroll
    for (int j = 0; j < kMaxTopkUnroll; ++j) {
      s[0] += v[j][0]; s[1] += v[j][1]; s[2] += v[j][2]; s[3] += v[j][3];
    }
  }
  for (; k < topk; ++k) {
    const f32x4_t w = load4<YDT>(src + (int64_t)k * H * ye);
    s[0] += w[0]; s[1] += w[1]; s[2] += w[2]; s[3] += w[3];
  }
  store4<CDT>(reinterpret_cast<uint8_t*>(out) + (t * H + c) * ElemBytes<CDT>::value,
              s[0], s[1], s[2], s[3]);
}

}  // namespace

hipError_t launch_moe_gemm_stream(const MoeGemmArgs& a, hipStream_t stream) {
  return a.block_m == 16 ? launch_tg<1>(a, stream) : launch_tg<2>(a, stream);
}

hipError_t launch_topk_reduce(const void* y, int y_dtype, int64_t T, int topk, int64_t H,
                              void* out, int out_dtype, hipStream_t stream) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
#define MOE_REDUCE(YD, CD) \
  hipLaunchKernelGGL((topk_reduce_kernel<YD, CD>), grid, block, 0, stream, y, T, topk, H, out)
  if (y_dtype == 0) {
    if (out_dtype == 0) MOE_REDUCE(0, 0);
    else if (out_dtype == 1) MOE_REDUCE(0, 1);
    else MOE_REDUCE(0, 2);
  } else {
    if (out_dtype == 0) MOE_REDUCE(1, 0);
    else if (out_dtype == 1) MOE_REDUCE(1, 1);
    else MOE_REDUCE(1, 2);
  }
#undef MOE_REDUCE
  return hipGetLastError();
}

}  // namespace moe

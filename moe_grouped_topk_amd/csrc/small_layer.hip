// Whole MoE layer for problems small enough that kernel launches, not work,
// set its latency (the tiny layer: T = 64, H = 128, I = 256, E = 8, top-2).
// After routing, one launch does the rest of moe_forward's pipeline, token by
// token ("mini-sglang: MoE and fused MoE", the per-token form of the layer):
// workgroup t walks its token's top-k pairs in k order and, for each,
//   h = silu(x W1[e][gate]^T) * (x W1[e][up]^T)      (fp32, in LDS)
//   out[t] += w * (h W2[e]^T)                         (fp32, in LDS)
// then writes out[t] in x's dtype.  A row's dot product is split over a team
// of lanes (16-byte weight pieces, coalesced) and summed by shuffles.  x is
// used in fp32 as given (the MFMA path rounds it to bf16) and h stays fp32;
// nothing crosses workgroups, so the result is deterministic.  The weights
// of the few experts stay in L2 for all workgroups.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kSmallThreads = 1024;
constexpr int kSmallRowsPerTeam = 4;   // rows a team works on at once (loads in flight)
constexpr int kSmallMaxPairs = 2048;
constexpr double kSmallMaxFlops = 268435456.0;   // 6 * pairs * H * I at most

template <int XDT>
__device__ __forceinline__ float load_x(const void* x, int64_t i) {
  if constexpr (XDT == 0) {
    return reinterpret_cast<const float*>(x)[i];
  } else {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
  }
}

// Lanes per row: the largest power of two <= min(64, row length / 8).
__device__ __forceinline__ int team_lanes(int len) {
  int tl = 1;
  while (tl * 2 <= kWave && tl * 2 <= len / 8) tl *= 2;
  return tl;
}

// Dot product of 8 bf16 (16 bytes, already loaded) with 8 floats.
__device__ __forceinline__ float dot8(const u32x4_t& q, const float (&v)[8], float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc = fmaf(__uint_as_float(q[j] << 16), v[2 * j], acc);
    acc = fmaf(__uint_as_float(q[j] & 0xffff0000u), v[2 * j + 1], acc);
  }
  return acc;
}

__device__ __forceinline__ void lds8(const float* p, float (&v)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = p[j];
}

__device__ __forceinline__ float team_sum(float v, int tl) {
  for (int m = tl / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

template <int XDT>
__global__ void __launch_bounds__(kSmallThreads) small_layer_kernel(SmallLayerArgs a) {
  extern __shared__ float sm[];
  const int H = a.H, I = a.I;
  float* s_x = sm;            // [H] the token's row
  float* s_h = sm + H;        // [I]
  float* s_y = s_h + I;       // [H] output accumulator
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  for (int c = tid; c < H; c += kSmallThreads) {
    s_x[c] = load_x<XDT>(a.x, t * H + c);
    s_y[c] = 0.0f;
  }
  __syncthreads();
  const int tl1 = team_lanes(H), tl2 = team_lanes(I);
  const int nteam1 = kSmallThreads / tl1, team1 = tid / tl1, tlane1 = lane & (tl1 - 1);
  const int nteam2 = kSmallThreads / tl2, team2 = tid / tl2, tlane2 = lane & (tl2 - 1);
  for (int k = 0; k < a.topk; ++k) {
    const int64_t p = t * a.topk + k;
    const int e = a.ids[p];
    const float w = a.w[p];
    const uint16_t* W1 = reinterpret_cast<const uint16_t*>(a.w1) + (int64_t)e * 2 * I * H;
    const uint16_t* W2 = reinterpret_cast<const uint16_t*>(a.w2) + (int64_t)e * H * I;
    // gate and up rows: each team takes kSmallRowsPerTeam rows at once, its
    // lanes splitting the row; past the last row a team re-reads row I - 1
    constexpr int R = kSmallRowsPerTeam;
    for (int i0 = 0; i0 < I; i0 += R * nteam1) {
      float g[R], u[R];
      const uint16_t* wg[R];
      const uint16_t* wu[R];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        int i = i0 + team1 + j * nteam1;
        i = i < I ? i : I - 1;
        wg[j] = W1 + (int64_t)i * H;
        wu[j] = W1 + (int64_t)(I + i) * H;
        g[j] = 0.0f;
        u[j] = 0.0f;
      }
      for (int c = tlane1 * 8; c < H; c += tl1 * 8) {
        u32x4_t qg[R], qu[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          qg[j] = *reinterpret_cast<const u32x4_t*>(wg[j] + c);
          qu[j] = *reinterpret_cast<const u32x4_t*>(wu[j] + c);
        }
        float xv[8];
        lds8(s_x + c, xv);
#pragma unroll
        for (int j = 0; j < R; ++j) {
          g[j] = dot8(qg[j], xv, g[j]);
          u[j] = dot8(qu[j], xv, u[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float gs = team_sum(g[j], tl1), us = team_sum(u[j], tl1);
        const int i = i0 + team1 + j * nteam1;
        if (i < I && tlane1 == 0) s_h[i] = silu_f32(gs) * us;
      }
    }
    __syncthreads();
    // down rows, times the routing weight, added in k order
    for (int c0 = 0; c0 < H; c0 += R * nteam2) {
      float y[R];
      const uint16_t* w2[R];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        int c = c0 + team2 + j * nteam2;
        c = c < H ? c : H - 1;
        w2[j] = W2 + (int64_t)c * I;
        y[j] = 0.0f;
      }
      for (int i = tlane2 * 8; i < I; i += tl2 * 8) {
        u32x4_t q[R];
#pragma unroll
        for (int j = 0; j < R; ++j) q[j] = *reinterpret_cast<const u32x4_t*>(w2[j] + i);
        float hv[8];
        lds8(s_h + i, hv);
#pragma unroll
        for (int j = 0; j < R; ++j) y[j] = dot8(q[j], hv, y[j]);
      }
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float ys = team_sum(y[j], tl2);
        const int c = c0 + team2 + j * nteam2;
        if (c < H && tlane2 == 0) s_y[c] += w * ys;
      }
    }
    __syncthreads();
  }
  for (int c = tid; c < H; c += kSmallThreads) {
    if constexpr (XDT == 0) {
      reinterpret_cast<float*>(a.out)[t * H + c] = s_y[c];
    } else {
      reinterpret_cast<uint16_t*>(a.out)[t * H + c] = (uint16_t)(pack_bf16x2(s_y[c], 0.0f) & 0xffffu);
    }
  }
}

}  // namespace

bool small_layer_fits(int64_t T, int H, int I, int E, int topk) {
  const int64_t P = T * topk;
  if (P < 1 || P > kSmallMaxPairs || T > INT32_MAX) return false;
  if (H % 8 != 0 || I % 8 != 0 || H > 4096 || I > 4096) return false;
  (void)E;
  return 6.0 * (double)P * H * I <= kSmallMaxFlops;
}

hipError_t launch_small_layer(const SmallLayerArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)(2 * a.H + a.I) * sizeof(float);
  const dim3 grid((unsigned)a.T), block(kSmallThreads);
  if (a.x_dtype == 0)
    hipLaunchKernelGGL(small_layer_kernel<0>, grid, block, lds, stream, a);
  else
    hipLaunchKernelGGL(small_layer_kernel<1>, grid, block, lds, stream, a);
  return hipGetLastError();
}

}  // namespace moe

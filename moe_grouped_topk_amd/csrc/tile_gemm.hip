// MFMA tile kernels: the sorted grouped GEMM of the fused MoE (bf16) and the
// INT8 grouped GEMM (GMM).
//
// Semantics: mini-sglang "MoE and fused MoE", fused_moe_kernel (one output
// block per program, one expert per block, A rows gathered through the sorted
// pair list, placeholder rows masked, optional routing-weight multiply) with
// the SiLU(gate)*up epilogue of that page's exercise 3; the GMM of the
// low-precision GMM article, sections 2.1 / 3.1 (rows grouped by offsets,
// per-row and per-channel scales, int32 accumulation per section 5.3).
//
// gfx950 design (not the pages' Triton tiling):
//  * 256 threads = 4 wave64s in a 2 (weight rows) x 2 (tokens) grid.  A tile
//    is BN weight rows x BM tokens (BN 128/256, BM 64/128/256); a wave owns
//    BN/2 x BM/2 and computes it with v_mfma_f32_32x32x16_bf16 (or
//    v_mfma_i32_32x32x32_i8) blocks.  At BN = BM = 256 a wave holds a
//    128 x 128 fp32 accumulator (256 registers, kept in AGPRs), which halves
//    the LDS operand traffic per FLOP of a 64 x 64 wave tile.
//  * Operands are swapped relative to the usual C = A.B^T picture: weight
//    rows sit in the MFMA's row slot and tokens in its column slot, so each
//    lane ends up with runs of 4 consecutive OUTPUT FEATURES of one token:
//    packed stores, and gate and up (or a channel scale) in the same lane.
//  * K advances 128 bytes per stage (64 bf16 or 128 int8 = 4 MFMA k-steps).
//    Global -> registers -> LDS with two LDS stages and two register
//    buffers: the loads of stage k+2 are issued before the MFMAs of stage k,
//    so two stages of loads are in flight while the matrix cores run.  LDS
//    rows are padded to 144 bytes, which makes every group of 8 lanes reading
//    16 bytes hit 8 distinct bank quads.
//  * Token rows are gathered straight from x into LDS by pair index; the
//    gathered tensor never exists in HBM.  Placeholder rows load nothing
//    (zeros) and 32-token column blocks with no valid row skip their MFMAs.
//  * Tiles are numbered block-major (all n-tiles of a block adjacent, the
//    blocks of one expert adjacent), and xcd_remap gives each XCD one
//    contiguous run of tiles, so an expert's weight slab and its gathered
//    rows are shared in one XCD's L2.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kBKB = 128;             // K bytes per stage
constexpr int kLdsRow = kBKB + 16;    // padded LDS row, bytes
constexpr int kMaxGmmExperts = 1024;

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int i32x16_t;

template <int BN, int BM>
struct Shape {
  static constexpr int RB = BN / 64;   // 32-row weight blocks per wave
  static constexpr int CB = BM / 64;   // 32-token blocks per wave
  static constexpr int WR = BN / 32;   // weight rows staged per thread per stage
  static constexpr int TR = BM / 32;   // token rows staged per thread per stage
  static constexpr int kStage = (BN + BM) * kLdsRow;
  static constexpr int kBytes = 2 * kStage;
};

template <int KIND> struct Mma;
template <> struct Mma<0> {   // bf16 x bf16 -> f32
  typedef f32x16_t acc_t;
  static __device__ __forceinline__ acc_t run(const u32x4_t& a, const u32x4_t& b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<1> {   // int8 x int8 -> int32 (exact)
  typedef i32x16_t acc_t;
  static __device__ __forceinline__ acc_t run(const u32x4_t& a, const u32x4_t& b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4_t, a),
                                                 __builtin_bit_cast(i32x4_t, b), c, 0, 0, 0);
  }
};

__device__ __forceinline__ u32x4_t cvt_f32x8_bf16(const u32x4_t& lo, const u32x4_t& hi) {
  u32x4_t r;
  r[0] = pack_bf16x2(__uint_as_float(lo[0]), __uint_as_float(lo[1]));
  r[1] = pack_bf16x2(__uint_as_float(lo[2]), __uint_as_float(lo[3]));
  r[2] = pack_bf16x2(__uint_as_float(hi[0]), __uint_as_float(hi[1]));
  r[3] = pack_bf16x2(__uint_as_float(hi[2]), __uint_as_float(hi[3]));
  return r;
}

// Where this thread's staged rows come from.
//   weight row i (local row lrow + 32 i): (i < WR/2 ? w0 : w1) + (i % (WR/2)) * wstep,
//     loaded only if bit i of wmask is set;
//   token row i (local row lrow + 32 i): abase + trow[i] * arow_bytes, if trow[i] >= 0.
template <int BN, int BM>
struct Src {
  const uint8_t* w0;
  const uint8_t* w1;
  int64_t wstep;
  uint32_t wmask;
  const uint8_t* abase;
  int64_t arow_bytes;
  int trow[Shape<BN, BM>::TR];
};

template <int BN, int BM, bool TF32>
struct Stage {
  u32x4_t w[Shape<BN, BM>::WR];
  u32x4_t t[Shape<BN, BM>::TR][TF32 ? 2 : 1];
};

// The K loop shared by both kernels.
//   kbytes  : bytes of K in a weight row (float32 token rows hold twice that).
//   wrow[rb]: first local weight row of this wave's 32-row block rb.
//   tcol0   : first local token row of this wave.
//   active  : bit cb set if token block cb of this wave holds a valid row.
template <int BN, int BM, int KIND, bool TF32>
__device__ __forceinline__ void mainloop(uint8_t* smem, const Src<BN, BM>& src, int64_t kbytes,
                                         const int (&wrow)[Shape<BN, BM>::RB], int tcol0,
                                         uint32_t active,
                                         typename Mma<KIND>::acc_t (&acc)[Shape<BN, BM>::RB]
                                                                          [Shape<BN, BM>::CB]) {
  typedef Shape<BN, BM> S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int ch = tid & 7;
  const int lrow = tid >> 3;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  constexpr int HALF = S::WR / 2;

  auto gload = [&](Stage<BN, BM, TF32>& r, int kt) {
    const int64_t off = (int64_t)kt * kBKB + ch * 16;
    const bool kin = off < kbytes;
#pragma unroll
    for (int i = 0; i < S::WR; ++i) {
      const uint8_t* p = (i < HALF ? src.w0 : src.w1) + (int64_t)(i % HALF) * src.wstep + off;
      r.w[i] = (kin && ((src.wmask >> i) & 1u)) ? *reinterpret_cast<const u32x4_t*>(p) : zero;
    }
#pragma unroll
    for (int i = 0; i < S::TR; ++i) {
      const bool ok = kin && src.trow[i] >= 0;
      const uint8_t* p = src.abase + (int64_t)src.trow[i] * src.arow_bytes;
      if constexpr (TF32) {
        r.t[i][0] = ok ? *reinterpret_cast<const u32x4_t*>(p + 2 * off) : zero;
        r.t[i][1] = ok ? *reinterpret_cast<const u32x4_t*>(p + 2 * off + 16) : zero;
      } else {
        r.t[i][0] = ok ? *reinterpret_cast<const u32x4_t*>(p + off) : zero;
      }
    }
  };
  auto sstore = [&](const Stage<BN, BM, TF32>& r, int buf) {
    uint8_t* base = smem + buf * S::kStage + lrow * kLdsRow + ch * 16;
#pragma unroll
    for (int i = 0; i < S::WR; ++i)
      *reinterpret_cast<u32x4_t*>(base + 32 * i * kLdsRow) = r.w[i];
#pragma unroll
    for (int i = 0; i < S::TR; ++i) {
      u32x4_t v;
      if constexpr (TF32) v = cvt_f32x8_bf16(r.t[i][0], r.t[i][1]);
      else v = r.t[i][0];
      *reinterpret_cast<u32x4_t*>(base + (BN + 32 * i) * kLdsRow) = v;
    }
  };
  auto mma = [&](int buf) {
    const uint8_t* base = smem + buf * S::kStage + (lane & 31) * kLdsRow + (lane >> 5) * 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t af[S::RB];
#pragma unroll
      for (int rb = 0; rb < S::RB; ++rb)
        af[rb] = *reinterpret_cast<const u32x4_t*>(base + wrow[rb] * kLdsRow + ks * 32);
#pragma unroll
      for (int cb = 0; cb < S::CB; ++cb) {
        if (!((active >> cb) & 1u)) continue;
        const u32x4_t bf = *reinterpret_cast<const u32x4_t*>(
            base + (BN + tcol0 + cb * 32) * kLdsRow + ks * 32);
#pragma unroll
        for (int rb = 0; rb < S::RB; ++rb) acc[rb][cb] = Mma<KIND>::run(af[rb], bf, acc[rb][cb]);
      }
    }
  };

  const int nk = (int)((kbytes + kBKB - 1) / kBKB);
  Stage<BN, BM, TF32> r0, r1;
  gload(r0, 0);
  if (nk > 1) gload(r1, 1);
  sstore(r0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // stage kt is in LDS buffer 0, stage kt+1 is landing in r1
    if (kt + 2 < nk) gload(r0, kt + 2);
    mma(0);
    if (kt + 1 < nk) sstore(r1, 1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    // stage kt+1 is in LDS buffer 1, stage kt+2 is landing in r0
    if (kt + 3 < nk) gload(r1, kt + 3);
    mma(1);
    if (kt + 2 < nk) sstore(r0, 0);
    __syncthreads();
  }
}

template <int CB>
__device__ __forceinline__ uint32_t active_blocks(const int* rowinfo, int tcol0) {
  const int lane = threadIdx.x & 63;
  uint32_t active = 0u;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const bool v = rowinfo[tcol0 + cb * 32 + (lane & 31)] >= 0;
    if (__ballot(v) != 0ull) active |= 1u << cb;
  }
  return active;
}

// ---------------------------------------------------------------------------
// Fused-MoE grouped GEMM (bf16 weights, MFMA bf16 -> f32).
//   EPI 0: C = acc;  EPI 1: C[:, j] = silu(acc_gate_j) * acc_up_j.
//   TF32: tokens are float32 rows (rounded to bf16 on the way to LDS).
template <int BN, int BM, int EPI, bool TF32, int CDT>
__global__ void __launch_bounds__(kThreads) moe_gemm_tile_kernel(MoeGemmArgs a) {
  typedef Shape<BN, BM> S;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int rowinfo[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int64_t ncols = EPI ? BN / 2 : BN;            // output columns per tile
  const int ntile = (int)((Nout + ncols - 1) / ncols);
  const int nblk = *a.total / BM;
  const int live = nblk * ntile;
  if ((int)blockIdx.x >= live) return;
  const int L = xcd_remap((int)blockIdx.x, live);
  const int blk = L / ntile, nt = L % ntile;
  const int e = a.expert_ids[blk];
  if (e < 0) return;
  const int64_t s0 = (int64_t)blk * BM;
  const int64_t c0 = (int64_t)nt * ncols;

  if (tid < BM) {
    const int p = a.sorted_ids[s0 + tid];
    rowinfo[tid] = (p >= 0 && p < a.num_valid) ? p : -1;
  }
  __syncthreads();

  const int lrow = tid >> 3;
  const int64_t wrow_bytes = a.K * 2;
  const uint8_t* Bw = reinterpret_cast<const uint8_t*>(a.B) + (int64_t)e * a.N * wrow_bytes;
  Src<BN, BM> src;
  constexpr int HALF = S::WR / 2;
  src.wstep = 32 * wrow_bytes;
  src.wmask = 0u;
  if (EPI) {
    src.w0 = Bw + (c0 + lrow) * wrow_bytes;            // gate row c0 + lrow
    src.w1 = Bw + (Nout + c0 + lrow) * wrow_bytes;     // up row
#pragma unroll
    for (int i = 0; i < S::WR; ++i)
      if (c0 + lrow + 32 * (i % HALF) < Nout) src.wmask |= 1u << i;
  } else {
    src.w0 = Bw + (c0 + lrow) * wrow_bytes;
    src.w1 = src.w0 + HALF * src.wstep;
#pragma unroll
    for (int i = 0; i < S::WR; ++i)
      if (c0 + lrow + 32 * i < a.N) src.wmask |= 1u << i;
  }
  src.abase = reinterpret_cast<const uint8_t*>(a.A);
  src.arow_bytes = a.lda * (TF32 ? 4 : 2);
#pragma unroll
  for (int i = 0; i < S::TR; ++i) {
    const int r = lrow + 32 * i;
    const int p = rowinfo[r];
    src.trow[i] = p < 0 ? -1 : (a.a_rows == 0 ? p / a.a_row_div : (int)(s0 + r));
  }

  int wrow[S::RB];
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
    wrow[rb] = EPI ? ((rb < S::RB / 2) ? wn * (BN / 4) + rb * 32
                                       : BN / 2 + wn * (BN / 4) + (rb - S::RB / 2) * 32)
                   : wn * (BN / 2) + rb * 32;
  const int tcol0 = wm * (BM / 2);
  const uint32_t active = active_blocks<S::CB>(rowinfo, tcol0);

  f32x16_t acc[S::RB][S::CB];
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;

  mainloop<BN, BM, 0, TF32>(smem, src, wrow_bytes, wrow, tcol0, active, acc);

  // Epilogue.  32x32 MFMA output: lane holds token column (lane & 31) and,
  // for g = 0..3, rows 8 g + 4 (lane >> 5) + [0, 4) of its 32-row block.
  uint8_t* Cb = reinterpret_cast<uint8_t*>(a.C);
  constexpr int ce = ElemBytes<CDT>::value;
  const int rsub = 4 * (lane >> 5);
#pragma unroll
  for (int cb = 0; cb < S::CB; ++cb) {
    if (!((active >> cb) & 1u)) continue;
    const int trow = tcol0 + cb * 32 + (lane & 31);
    const int p = rowinfo[trow];
    if (p < 0) continue;
    const int64_t crow = (a.c_rows == 0) ? (int64_t)p : s0 + trow;
    const float w = a.topk_weights ? a.topk_weights[p] : 1.0f;
    uint8_t* rowp = Cb + crow * a.ldc * ce;
    if (EPI) {
#pragma unroll
      for (int j = 0; j < S::RB / 2; ++j) {
        const f32x16_t gt = acc[j][cb], up = acc[j + S::RB / 2][cb];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = c0 + wn * (BN / 4) + j * 32 + 8 * g + rsub;
          if (col < Nout)
            store4<CDT>(rowp + col * ce, silu_f32(gt[4 * g]) * up[4 * g] * w,
                        silu_f32(gt[4 * g + 1]) * up[4 * g + 1] * w,
                        silu_f32(gt[4 * g + 2]) * up[4 * g + 2] * w,
                        silu_f32(gt[4 * g + 3]) * up[4 * g + 3] * w);
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < S::RB; ++rb) {
        const f32x16_t v = acc[rb][cb];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = c0 + wrow[rb] + 8 * g + rsub;
          if (col < a.N)
            store4<CDT>(rowp + col * ce, v[4 * g] * w, v[4 * g + 1] * w, v[4 * g + 2] * w,
                        v[4 * g + 3] * w);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// INT8 GMM: rows [off[e], off[e+1]) of X use W[e]; fp16 output.
constexpr int kGmmBN = 256;
constexpr int kGmmBM = 128;

__global__ void __launch_bounds__(kThreads) gmm_i8_tile_kernel(GmmI8Args a) {
  constexpr int BN = kGmmBN, BM = kGmmBM;
  typedef Shape<BN, BM> S;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int tprefix[kMaxGmmExperts + 1];   // m-tiles before expert e
  __shared__ int scan_buf[kThreads];
  __shared__ int rowinfo[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int E = a.E;
  const int M = (int)a.M;
  const int ntile = (int)((a.N + BN - 1) / BN);

  // m-tile counts per expert from the (clamped) offsets, then a scan.
  auto lo_of = [&](int e) {
    int v = a.offsets[e];
    return v < 0 ? 0 : (v > M ? M : v);
  };
  const int per = (E + kThreads - 1) / kThreads;   // <= 4
  int cnt[4] = {0, 0, 0, 0};
  int local = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid * per + j;
    if (j < per && e < E) {
      const int lo = lo_of(e);
      int hi = lo_of(e + 1);
      hi = hi < lo ? lo : hi;
      cnt[j] = (hi - lo + BM - 1) / BM;
      local += cnt[j];
    }
  }
  scan_buf[tid] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int add = tid >= off ? scan_buf[tid - off] : 0;
    __syncthreads();
    scan_buf[tid] += add;
    __syncthreads();
  }
  {
    int run = scan_buf[tid] - local;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid * per + j;
      if (j < per && e < E) {
        tprefix[e] = run;
        run += cnt[j];
      }
    }
    if (tid == kThreads - 1) tprefix[E] = scan_buf[tid];
  }
  __syncthreads();
  const int total_mt = tprefix[E];
  const int live = total_mt * ntile;
  if ((int)blockIdx.x >= live) return;
  const int L = xcd_remap((int)blockIdx.x, live);
  // Expert: largest e with tprefix[e] * ntile <= L.
  int lo = 0, hi = E;   // invariant: tprefix[lo]*ntile <= L < tprefix[hi]*ntile
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tprefix[mid] * ntile <= L) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int mcount = tprefix[e + 1] - tprefix[e];
  const int lin = L - tprefix[e] * ntile;
  const int nt = lin / mcount, mt = lin % mcount;   // m-tiles of one n-tile adjacent
  const int row_lo = lo_of(e);
  int row_hi = lo_of(e + 1);
  row_hi = row_hi < row_lo ? row_lo : row_hi;
  const int row0 = row_lo + mt * BM;
  const int64_t n0 = (int64_t)nt * BN;

  if (tid < BM) rowinfo[tid] = (row0 + tid < row_hi) ? row0 + tid : -1;
  __syncthreads();

  const int lrow = tid >> 3;
  Src<BN, BM> src;
  constexpr int HALF = S::WR / 2;
  src.wstep = 32 * a.K;
  src.w0 = reinterpret_cast<const uint8_t*>(a.W) + ((int64_t)e * a.N + n0 + lrow) * a.K;
  src.w1 = src.w0 + HALF * src.wstep;
  src.wmask = 0u;
#pragma unroll
  for (int i = 0; i < S::WR; ++i)
    if (n0 + lrow + 32 * i < a.N) src.wmask |= 1u << i;
  src.abase = reinterpret_cast<const uint8_t*>(a.X);
  src.arow_bytes = a.K;
#pragma unroll
  for (int i = 0; i < S::TR; ++i) src.trow[i] = rowinfo[lrow + 32 * i];

  int wrow[S::RB];
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb) wrow[rb] = wn * (BN / 2) + rb * 32;
  const int tcol0 = wm * (BM / 2);
  const uint32_t active = active_blocks<S::CB>(rowinfo, tcol0);

  i32x16_t acc[S::RB][S::CB];
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0;

  mainloop<BN, BM, 1, false>(smem, src, a.K, wrow, tcol0, active, acc);

  uint8_t* Yb = reinterpret_cast<uint8_t*>(a.Y);
  const int rsub = 4 * (lane >> 5);
#pragma unroll
  for (int cb = 0; cb < S::CB; ++cb) {
    if (!((active >> cb) & 1u)) continue;
    const int m = rowinfo[tcol0 + cb * 32 + (lane & 31)];
    if (m < 0) continue;
    const float sx = a.sx[m];
#pragma unroll
    for (int rb = 0; rb < S::RB; ++rb) {
      const i32x16_t v = acc[rb][cb];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wrow[rb] + 8 * g + rsub;
        if (n < a.N) {
          const f32x4_t sw = *reinterpret_cast<const f32x4_t*>(a.sw + (int64_t)e * a.N + n);
          store4<2>(Yb + ((int64_t)m * a.N + n) * 2, (float)v[4 * g] * sx * sw[0],
                    (float)v[4 * g + 1] * sx * sw[1], (float)v[4 * g + 2] * sx * sw[2],
                    (float)v[4 * g + 3] * sx * sw[3]);
        }
      }
    }
  }
}

// Dynamic LDS beyond 64 KiB has to be requested per kernel.
template <typename K>
hipError_t ensure_lds(K kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <int BN, int BM, int EPI, bool TF32, int CDT>
hipError_t launch_tile_t(const MoeGemmArgs& a, hipStream_t stream) {
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int64_t ncols = EPI ? BN / 2 : BN;
  const int64_t ntile = (Nout + ncols - 1) / ncols;
  const int64_t grid = (a.max_padded / BM) * ntile;
  if (grid == 0) return hipSuccess;
  auto k = moe_gemm_tile_kernel<BN, BM, EPI, TF32, CDT>;
  constexpr size_t lds = Shape<BN, BM>::kBytes;
  const hipError_t st = ensure_lds(k, lds);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int BN, int BM, int EPI, bool TF32>
hipError_t launch_tile_c(const MoeGemmArgs& a, hipStream_t s) {
  switch (a.c_dtype) {
    case 0: return launch_tile_t<BN, BM, EPI, TF32, 0>(a, s);
    case 1: return launch_tile_t<BN, BM, EPI, TF32, 1>(a, s);
    default: return launch_tile_t<BN, BM, EPI, TF32, 2>(a, s);
  }
}

template <int BM>
hipError_t launch_tile_bm(const MoeGemmArgs& a, hipStream_t s) {
  constexpr int BN = 256;
  const bool tf32 = a.a_dtype == 0;
  if constexpr (BM > 128) {
    if (tf32) return hipErrorInvalidValue;   // rejected by the ABI layer beforehand
    return a.epilogue ? launch_tile_c<BN, BM, 1, false>(a, s) : launch_tile_c<BN, BM, 0, false>(a, s);
  } else {
    if (a.epilogue)
      return tf32 ? launch_tile_c<BN, BM, 1, true>(a, s) : launch_tile_c<BN, BM, 1, false>(a, s);
    return tf32 ? launch_tile_c<BN, BM, 0, true>(a, s) : launch_tile_c<BN, BM, 0, false>(a, s);
  }
}

}  // namespace

hipError_t launch_moe_gemm_tile(const MoeGemmArgs& a, hipStream_t stream) {
  switch (a.block_m) {
    case 64: return launch_tile_bm<64>(a, stream);
    case 128: return launch_tile_bm<128>(a, stream);
    default: return launch_tile_bm<256>(a, stream);
  }
}

hipError_t launch_gmm_int8(const GmmI8Args& a, hipStream_t stream) {
  const int ntile = (int)((a.N + kGmmBN - 1) / kGmmBN);
  // Upper bound of m-tiles: every non-empty expert adds at most one partial tile.
  const int64_t mt_max = (a.M + kGmmBM - 1) / kGmmBM + a.E;
  const int64_t grid = mt_max * ntile;
  if (grid == 0 || a.M == 0) return hipSuccess;
  typedef Shape<kGmmBN, kGmmBM> S;
  const hipError_t st = ensure_lds(gmm_i8_tile_kernel, S::kBytes);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(gmm_i8_tile_kernel, dim3((unsigned)grid), dim3(kThreads), S::kBytes, stream,
                     a);
  return hipGetLastError();
}

}  // namespace moe

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
//  * 256 threads = 4 wave64s in a 2 (weight rows) x 2 (token rows) grid.
//    A tile is 128 weight rows x BM token rows; each wave owns 64 x BM/2.
//  * Operands are swapped relative to the usual C = A.B^T picture: the
//    weight rows occupy the 16-row slot of v_mfma_*_16x16x32_bf16 /
//    v_mfma_i32_16x16x64_i8 and the tokens the 16-column slot.  Each lane
//    then ends up with 4 consecutive OUTPUT FEATURES of one token, which
//    gives packed 8/16-byte stores and keeps gate and up (or a scale) in the
//    same lane for the epilogue.
//  * K advances 128 bytes per stage (64 bf16 or 128 int8 = 2 MFMA steps).
//    Global -> registers -> LDS with two LDS stages; the next stage's global
//    loads are in flight while the current stage's MFMAs run.  LDS rows are
//    padded to 144 bytes so each group of 8 lanes reading 16 bytes hits 8
//    distinct bank quads.
//  * Token rows are gathered straight from x into LDS by pair index; the
//    gathered tensor never exists in HBM.  Placeholder rows load nothing
//    (zeros) and 16-token column blocks with no valid row skip their MFMAs.
//  * Tiles are numbered so that all tiles of one expert are consecutive,
//    and xcd_remap gives each XCD one contiguous run of tiles, so an
//    expert's weight slab and gathered rows are shared in one L2.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kBN = 128;              // weight rows per tile
constexpr int kBKB = 128;             // K bytes per stage
constexpr int kLdsRow = kBKB + 16;    // padded LDS row, bytes
constexpr int kMaxGmmExperts = 1024;

template <int BM>
struct Smem {
  static constexpr int kStage = (kBN + BM) * kLdsRow;
  static constexpr int kBytes = 2 * kStage;
};

// MFMA on 16-byte operand fragments.
template <int KIND> struct Mma;
template <> struct Mma<0> {   // bf16 -> f32
  typedef f32x4_t acc_t;
  static __device__ __forceinline__ acc_t run(const u32x4_t& a, const u32x4_t& b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<1> {   // int8 -> int32 (exact)
  typedef i32x4_t acc_t;
  static __device__ __forceinline__ acc_t run(const u32x4_t& a, const u32x4_t& b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4_t, a),
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

// The K loop shared by both kernels.
//   wp[i]   : weight row base of local weight row (tid>>3) + 32 i, or null.
//   tp[i]   : token row base of local token row (tid>>3) + 32 i, or null.
//   kbytes  : bytes of K in a weight row (token rows: same, or twice that
//             for float32 tokens, TF32 = true).
//   wrow[rb]: first local weight row of this wave's row block rb.
//   active  : bit cb set if token column block cb of this wave has a valid row.
template <int BM, int KIND, bool TF32>
__device__ __forceinline__ void mainloop(uint8_t* smem, const uint8_t* const (&wp)[4],
                                         const uint8_t* const (&tp)[BM / 32], int64_t kbytes,
                                         const int (&wrow)[4], int tcol0, uint32_t active,
                                         typename Mma<KIND>::acc_t (&acc)[4][BM / 32]) {
  constexpr int NCB = BM / 32;     // token column blocks per wave (BM/2 tokens)
  constexpr int TR = BM / 32;      // token rows staged per thread
  const int tid = threadIdx.x, lane = tid & 63;
  const int ch = tid & 7;
  const int lrow = tid >> 3;
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  u32x4_t wreg[4];
  u32x4_t treg[TR][TF32 ? 2 : 1];

  auto gload = [&](int kt) {
    const int64_t off = (int64_t)kt * kBKB + ch * 16;
    const bool kin = off < kbytes;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wreg[i] = (wp[i] && kin) ? *reinterpret_cast<const u32x4_t*>(wp[i] + off) : zero;
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      if constexpr (TF32) {
        const bool ok = tp[i] && kin;
        treg[i][0] = ok ? *reinterpret_cast<const u32x4_t*>(tp[i] + 2 * off) : zero;
        treg[i][1] = ok ? *reinterpret_cast<const u32x4_t*>(tp[i] + 2 * off + 16) : zero;
      } else {
        treg[i][0] = (tp[i] && kin) ? *reinterpret_cast<const u32x4_t*>(tp[i] + off) : zero;
      }
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * Smem<BM>::kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t*>(base + (lrow + 32 * i) * kLdsRow + ch * 16) = wreg[i];
#pragma unroll
    for (int i = 0; i < TR; ++i) {
      u32x4_t v;
      if constexpr (TF32) v = cvt_f32x8_bf16(treg[i][0], treg[i][1]);
      else v = treg[i][0];
      *reinterpret_cast<u32x4_t*>(base + (kBN + lrow + 32 * i) * kLdsRow + ch * 16) = v;
    }
  };
  auto mma = [&](int buf) {
    const uint8_t* base = smem + buf * Smem<BM>::kStage;
    const int fo = (lane >> 4) * 16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4_t af[4];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        af[rb] = *reinterpret_cast<const u32x4_t*>(base + (wrow[rb] + (lane & 15)) * kLdsRow +
                                                   ks * 64 + fo);
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        if (!((active >> cb) & 1u)) continue;
        const int trow = tcol0 + cb * 16 + (lane & 15);
        const u32x4_t bf =
            *reinterpret_cast<const u32x4_t*>(base + (kBN + trow) * kLdsRow + ks * 64 + fo);
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) acc[rb][cb] = Mma<KIND>::run(af[rb], bf, acc[rb][cb]);
      }
    }
  };

  const int nk = (int)((kbytes + kBKB - 1) / kBKB);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    mma(cur);
    if (more) sstore(cur ^ 1);
    __syncthreads();
  }
}

template <int BM>
__device__ __forceinline__ uint32_t active_blocks(const int* rowinfo, int tcol0) {
  const int lane = threadIdx.x & 63;
  uint32_t active = 0u;
#pragma unroll
  for (int cb = 0; cb < BM / 32; ++cb) {
    const bool v = rowinfo[tcol0 + cb * 16 + (lane & 15)] >= 0;
    if (__ballot(v) != 0ull) active |= 1u << cb;
  }
  return active;
}

// ---------------------------------------------------------------------------
// Fused-MoE grouped GEMM (bf16 weights, MFMA bf16 -> f32).
//   EPI 0: C = acc;  EPI 1: C[:, j] = silu(acc_gate_j) * acc_up_j.
//   TF32: tokens are float32 rows (rounded to bf16 on the way to LDS).
template <int BM, int EPI, bool TF32, int CDT>
__global__ void __launch_bounds__(kThreads, 2) moe_gemm_tile_kernel(MoeGemmArgs a) {
  constexpr int TR = BM / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int rowinfo[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int ntile = EPI ? (int)((Nout + 63) / 64) : (int)((a.N + kBN - 1) / kBN);
  const int nblk = *a.total / BM;
  const int live = nblk * ntile;
  if ((int)blockIdx.x >= live) return;
  const int L = xcd_remap((int)blockIdx.x, live);
  const int blk = L / ntile, nt = L % ntile;
  const int e = a.expert_ids[blk];
  if (e < 0) return;
  const int64_t s0 = (int64_t)blk * BM;

  if (tid < BM) {
    const int p = a.sorted_ids[s0 + tid];
    rowinfo[tid] = (p >= 0 && p < a.num_valid) ? p : -1;
  }
  __syncthreads();

  const int ch = tid & 7;
  (void)ch;
  const int lrow = tid >> 3;
  const uint8_t* Bw = reinterpret_cast<const uint8_t*>(a.B);
  const int64_t wrow_bytes = a.K * 2;
  const uint8_t* wp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 32 * i;
    int64_t grow;
    bool ok;
    if (EPI) {
      const int64_t hcol = (int64_t)nt * 64 + (r & 63);
      ok = hcol < Nout;
      grow = (r < 64) ? hcol : Nout + hcol;
    } else {
      grow = (int64_t)nt * kBN + r;
      ok = grow < a.N;
    }
    wp[i] = ok ? Bw + ((int64_t)e * a.N + grow) * wrow_bytes : nullptr;
  }
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(a.A);
  const int64_t a_row_bytes = a.lda * (TF32 ? 4 : 2);
  const uint8_t* tp[TR];
#pragma unroll
  for (int i = 0; i < TR; ++i) {
    const int r = lrow + 32 * i;
    const int p = rowinfo[r];
    const int64_t src = (a.a_rows == 0) ? (int64_t)(p / a.a_row_div) : s0 + r;
    tp[i] = (p >= 0) ? Ab + src * a_row_bytes : nullptr;
  }

  int wrow[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
    wrow[rb] = EPI ? ((rb < 2) ? wn * 32 + rb * 16 : 64 + wn * 32 + (rb - 2) * 16)
                   : wn * 64 + rb * 16;
  const int tcol0 = wm * (BM / 2);
  const uint32_t active = active_blocks<BM>(rowinfo, tcol0);

  f32x4_t acc[4][TR];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < TR; ++cb) acc[rb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  mainloop<BM, 0, TF32>(smem, wp, tp, wrow_bytes, wrow, tcol0, active, acc);

  // Epilogue: lane holds features 4*(lane>>4) + [0,4) of its row block for
  // token column (lane & 15) of each column block.
  uint8_t* Cb = reinterpret_cast<uint8_t*>(a.C);
  constexpr int ce = ElemBytes<CDT>::value;
#pragma unroll
  for (int cb = 0; cb < TR; ++cb) {
    if (!((active >> cb) & 1u)) continue;
    const int trow = tcol0 + cb * 16 + (lane & 15);
    const int p = rowinfo[trow];
    if (p < 0) continue;
    const int64_t crow = (a.c_rows == 0) ? (int64_t)p : s0 + trow;
    const float w = a.topk_weights ? a.topk_weights[p] : 1.0f;
    uint8_t* crow_ptr = Cb + crow * a.ldc * ce;
    if (EPI) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = (int64_t)nt * 64 + wn * 32 + j * 16 + 4 * (lane >> 4);
        if (col < Nout) {
          const f32x4_t g = acc[j][cb], u = acc[j + 2][cb];
          store4<CDT>(crow_ptr + col * ce, silu_f32(g[0]) * u[0] * w, silu_f32(g[1]) * u[1] * w,
                      silu_f32(g[2]) * u[2] * w, silu_f32(g[3]) * u[3] * w);
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int64_t col = (int64_t)nt * kBN + wn * 64 + rb * 16 + 4 * (lane >> 4);
        if (col < a.N) {
          const f32x4_t v = acc[rb][cb];
          store4<CDT>(crow_ptr + col * ce, v[0] * w, v[1] * w, v[2] * w, v[3] * w);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// INT8 GMM: rows [off[e], off[e+1]) of X use W[e]; fp16 output.
constexpr int kGmmBM = 128;

__global__ void __launch_bounds__(kThreads, 2) gmm_i8_tile_kernel(GmmI8Args a) {
  constexpr int BM = kGmmBM;
  constexpr int TR = BM / 32;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int tprefix[kMaxGmmExperts + 1];   // m-tiles before expert e
  __shared__ int scan_buf[kThreads];
  __shared__ int rowinfo[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 1, wm = wave >> 1;
  const int E = a.E;
  const int M = (int)a.M;
  const int ntile = (int)((a.N + kBN - 1) / kBN);

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
  // Find the expert: largest e with tprefix[e] * ntile <= L.
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

  if (tid < BM) rowinfo[tid] = (row0 + tid < row_hi) ? row0 + tid : -1;
  __syncthreads();

  const int lrow = tid >> 3;
  const uint8_t* wp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = (int64_t)nt * kBN + lrow + 32 * i;
    wp[i] = n < a.N ? reinterpret_cast<const uint8_t*>(a.W) + ((int64_t)e * a.N + n) * a.K : nullptr;
  }
  const uint8_t* tp[TR];
#pragma unroll
  for (int i = 0; i < TR; ++i) {
    const int m = rowinfo[lrow + 32 * i];
    tp[i] = m >= 0 ? reinterpret_cast<const uint8_t*>(a.X) + (int64_t)m * a.K : nullptr;
  }
  int wrow[4];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) wrow[rb] = wn * 64 + rb * 16;
  const int tcol0 = wm * (BM / 2);
  const uint32_t active = active_blocks<BM>(rowinfo, tcol0);

  i32x4_t acc[4][TR];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int cb = 0; cb < TR; ++cb) acc[rb][cb] = i32x4_t{0, 0, 0, 0};

  mainloop<BM, 1, false>(smem, wp, tp, a.K, wrow, tcol0, active, acc);

  uint8_t* Yb = reinterpret_cast<uint8_t*>(a.Y);
#pragma unroll
  for (int cb = 0; cb < TR; ++cb) {
    if (!((active >> cb) & 1u)) continue;
    const int m = rowinfo[tcol0 + cb * 16 + (lane & 15)];
    if (m < 0) continue;
    const float sx = a.sx[m];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int64_t n = (int64_t)nt * kBN + wn * 64 + rb * 16 + 4 * (lane >> 4);
      if (n < a.N) {
        const f32x4_t sw = *reinterpret_cast<const f32x4_t*>(a.sw + (int64_t)e * a.N + n);
        const i32x4_t v = acc[rb][cb];
        store4<2>(Yb + ((int64_t)m * a.N + n) * 2, (float)v[0] * sx * sw[0],
                  (float)v[1] * sx * sw[1], (float)v[2] * sx * sw[2], (float)v[3] * sx * sw[3]);
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

template <int BM, int EPI, bool TF32, int CDT>
hipError_t launch_tile_t(const MoeGemmArgs& a, hipStream_t stream) {
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int ntile = EPI ? (int)((Nout + 63) / 64) : (int)((a.N + kBN - 1) / kBN);
  const int64_t grid = (a.max_padded / BM) * ntile;
  if (grid == 0) return hipSuccess;
  auto k = moe_gemm_tile_kernel<BM, EPI, TF32, CDT>;
  const hipError_t st = ensure_lds(k, Smem<BM>::kBytes);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kThreads), Smem<BM>::kBytes, stream, a);
  return hipGetLastError();
}

template <int BM, int EPI, bool TF32>
hipError_t launch_tile_c(const MoeGemmArgs& a, hipStream_t s) {
  switch (a.c_dtype) {
    case 0: return launch_tile_t<BM, EPI, TF32, 0>(a, s);
    case 1: return launch_tile_t<BM, EPI, TF32, 1>(a, s);
    default: return launch_tile_t<BM, EPI, TF32, 2>(a, s);
  }
}

template <int BM>
hipError_t launch_tile_bm(const MoeGemmArgs& a, hipStream_t s) {
  const bool tf32 = a.a_dtype == 0;
  if (a.epilogue) return tf32 ? launch_tile_c<BM, 1, true>(a, s) : launch_tile_c<BM, 1, false>(a, s);
  return tf32 ? launch_tile_c<BM, 0, true>(a, s) : launch_tile_c<BM, 0, false>(a, s);
}

}  // namespace

hipError_t launch_moe_gemm_tile(const MoeGemmArgs& a, hipStream_t stream) {
  return a.block_m == 64 ? launch_tile_bm<64>(a, stream) : launch_tile_bm<128>(a, stream);
}

hipError_t launch_gmm_int8(const GmmI8Args& a, hipStream_t stream) {
  const int ntile = (int)((a.N + kBN - 1) / kBN);
  // Upper bound of m-tiles: every non-empty expert adds at most one partial tile.
  const int64_t mt_max = (a.M + kGmmBM - 1) / kGmmBM + a.E;
  const int64_t grid = mt_max * ntile;
  if (grid == 0 || a.M == 0) return hipSuccess;
  const hipError_t st = ensure_lds(gmm_i8_tile_kernel, Smem<kGmmBM>::kBytes);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(gmm_i8_tile_kernel, dim3((unsigned)grid), dim3(kThreads),
                     Smem<kGmmBM>::kBytes, stream, a);
  return hipGetLastError();
}

}  // namespace moe

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
//  * Operands are swapped relative to the usual C = A.B^T picture: weight
//    rows sit in the MFMA's row slot and tokens in its column slot, so each
//    lane ends up with runs of 4 consecutive OUTPUT FEATURES of one token
//    (v_mfma_f32_32x32x16_bf16 / v_mfma_i32_32x32x32_i8 blocks): packed
//    stores, and gate and up (or a channel scale) in the same lane.
//  * Token rows are gathered straight from x into LDS by pair index; the
//    gathered tensor never exists in HBM.  Placeholder rows are masked at
//    the store.
//  * Tile kernels (bf16 and int8 operands, moe_gemm_dma_kernel: decode and
//    experts with few rows; gmm_i8_tile_kernel): BN = 256 weight rows x BM =
//    64/128/256 tokens per tile, loaded with direct-to-LDS loads
//    (global_load_lds_dwordx4) into an NSTAGE ring of 64-byte K stages, with
//    no staging registers.  Weights may come pre-packed (moe_pack_weights) so
//    each wave's load is one contiguous, pre-swizzled 1 KiB piece.  Two
//    workgroups per CU at BM 64/128: one workgroup's MFMAs run while the
//    other waits for its loads.  Epilogues stage 16-bit output through LDS
//    and store whole 16-byte pieces of each output row.
//  * Expert-wide tiles (moe_gemm_wide_kernel: the prefill path, bf16 or
//    int8 operands): up to 10 token blocks (320 rows) of one expert against
//    256 weight rows, so each weight slice streams once per expert; one
//    persistent workgroup per CU; weight and token rings of their own (4 + 4
//    stages), loads issued between the MFMAs; the next tile's first weight
//    stages go out before the epilogue, which is staged in the LDS the next
//    tile does not use yet.
//  * float32 tokens (moe_gemm_tile_kernel): 4 waves in a 2 x 2 grid, global
//    -> registers (rounded to bf16) -> LDS with 128-byte K stages, LDS rows
//    padded to 144 bytes so every group of 8 lanes reading 16 bytes hits 8
//    distinct bank quads.
//  * Workgroups of a 1-D grid go to the 8 XCDs round-robin (id i to XCD
//    i % 8).  Tiles are numbered block-major (the n-tiles of a block
//    adjacent, the blocks of one expert adjacent).  The tile kernels hand
//    consecutive tiles to consecutive XCDs (each XCD streams a share of
//    every expert's weights); the expert-wide kernel gives each XCD one
//    contiguous run of tiles, so an expert's gathered rows are shared in one
//    XCD's L2; the GMM deals each expert's weight slices to the XCDs in turn.

#include "common.hpp"
#include "launch.hpp"

#include <atomic>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

namespace moe {

namespace {

constexpr int kBKB = 128;             // K bytes per stage
constexpr int kLdsRow = kBKB + 16;    // padded LDS row, bytes
constexpr int kMaxGmmExperts = 1024;

#ifndef MOE_TILE_NBUF
#define MOE_TILE_NBUF 1   // register prefetch buffers (loads one stage ahead)
#endif
#ifndef MOE_T256_WN
#define MOE_T256_WN 4     // 256 x 256 tile: 4 x 2 waves of 64 x 128
#define MOE_T256_WM 2
#endif
#ifndef MOE_T256_NSTAGE
#define MOE_T256_NSTAGE 4 // K stages in the LDS ring (4 x 32 KiB)
#endif


typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(16 * sizeof(int)))) int i32x16_t;

// Tile shape: BN weight rows x BM tokens, WN x WM waves (WN along the
// weight rows), NBUF register buffers for the global -> LDS staging.
template <int BN_, int BM_, int WN_, int WM_, int NBUF_>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, WN = WN_, WM = WM_, NBUF = NBUF_;
  static constexpr int THREADS = 64 * WN * WM;
  static constexpr int STEP = THREADS / 8;      // staged rows per pass (8 x 16 B per row)
  static constexpr int RB = BN / WN / 32;       // 32-row weight blocks per wave
  static constexpr int CB = BM / WM / 32;       // 32-token blocks per wave
  static constexpr int WR = BN / STEP;          // weight rows staged per thread per stage
  static constexpr int TR = BM / STEP;          // token rows staged per thread per stage
  static constexpr int kStage = (BN + BM) * kLdsRow;
  static constexpr int kBytes = 2 * kStage;
  static_assert(WR % 2 == 0 && TR >= 1 && RB >= 1 && CB >= 1, "tile shape");
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

// Where this thread's staged rows come from.  Every row address is
// dereferenceable: rows past the weight matrix and placeholder token rows
// read a valid row instead.  What they load only reaches output elements
// that the epilogue masks (an MFMA output element depends on one weight row
// and one token column only).  Loads are therefore unconditional, which
// keeps them out of branches and lets several stages stay in flight.
//   weight row i (local row lrow + STEP i) = w[i < WR/2 ? 0 : 1] + j * wstep with
//     j = min(i % (WR/2), wlast[...]); wlast < 0 means no valid row: w[0] is
//     then already a valid fallback row and j = 0;
//   token row i (local row lrow + STEP i) = abase + trow[i] * arow_bytes.
template <class C>
struct Src {
  const uint8_t* w[2];
  int64_t wstep;
  int wlast[2];
  const uint8_t* abase;
  int64_t arow_bytes;
  int trow[C::TR];
};

template <class C, bool TF32>
struct Stage {
  u32x4_t w[C::WR];
  u32x4_t t[C::TR][TF32 ? 2 : 1];
};

// The K loop shared by both kernels.
//   kbytes  : bytes of K in a weight row (float32 token rows hold twice that).
//   wrow[rb]: first local weight row of this wave's 32-row block rb.
//   tcol0   : first local token row of this wave.
// All MFMAs run, also on placeholder token columns (their outputs are never
// stored): a branch per column block would serialise the LDS reads with the
// MFMAs, and tiles that are mostly padding are bound by weight streaming.
template <class C, int KIND, bool TF32>
__device__ __forceinline__ void mainloop(uint8_t* smem, const Src<C>& src, int64_t kbytes,
                                         const int (&wrow)[C::RB], int tcol0,
                                         typename Mma<KIND>::acc_t (&acc)[C::RB][C::CB]) {
  typedef C S;
  constexpr int BN = C::BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int ch = tid & 7;
  const int lrow = tid >> 3;
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  constexpr int HALF = S::WR / 2;

  // K tail: a chunk past K loads from offset 0 of its row; it is zeroed when
  // written to LDS (a select at store time, when the data has arrived anyway).
  auto gload = [&](Stage<C, TF32>& r, int kt) {
    const int64_t off0 = (int64_t)kt * kBKB + ch * 16;
    const int64_t off = off0 < kbytes ? off0 : 0;
#pragma unroll
    for (int i = 0; i < S::WR; ++i) {
      const int h = i < HALF ? 0 : 1;
      const int j = i % HALF;
      const int jj = j < src.wlast[h] ? j : (src.wlast[h] < 0 ? 0 : src.wlast[h]);
      r.w[i] = *reinterpret_cast<const u32x4_t*>(src.w[h] + jj * src.wstep + off);
    }
#pragma unroll
    for (int i = 0; i < S::TR; ++i) {
      const uint8_t* t = src.abase + (int64_t)src.trow[i] * src.arow_bytes;
      if constexpr (TF32) {
        r.t[i][0] = *reinterpret_cast<const u32x4_t*>(t + 2 * off);
        r.t[i][1] = *reinterpret_cast<const u32x4_t*>(t + 2 * off + 16);
      } else {
        r.t[i][0] = *reinterpret_cast<const u32x4_t*>(t + off);
      }
    }
  };
  auto sstore = [&](const Stage<C, TF32>& r, int buf, int kt) {
    const bool kin = (int64_t)kt * kBKB + ch * 16 < kbytes;
    uint8_t* base = smem + buf * S::kStage + lrow * kLdsRow + ch * 16;
#pragma unroll
    for (int i = 0; i < S::WR; ++i)
      *reinterpret_cast<u32x4_t*>(base + S::STEP * i * kLdsRow) = kin ? r.w[i] : zero;
#pragma unroll
    for (int i = 0; i < S::TR; ++i) {
      u32x4_t v;
      if constexpr (TF32) v = cvt_f32x8_bf16(r.t[i][0], r.t[i][1]);
      else v = r.t[i][0];
      *reinterpret_cast<u32x4_t*>(base + (BN + S::STEP * i) * kLdsRow) = kin ? v : zero;
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
      u32x4_t bfr[S::CB];
#pragma unroll
      for (int cb = 0; cb < S::CB; ++cb)
        bfr[cb] = *reinterpret_cast<const u32x4_t*>(base + (BN + tcol0 + cb * 32) * kLdsRow +
                                                    ks * 32);
#pragma unroll
      for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
        for (int rb = 0; rb < S::RB; ++rb)
          acc[rb][cb] = Mma<KIND>::run(af[rb], bfr[cb], acc[rb][cb]);
    }
  };

  const int nk = (int)((kbytes + kBKB - 1) / kBKB);
  if constexpr (S::NBUF == 1) {
    // one register buffer: the loads of stage k+1 fly during the MFMAs of k
    Stage<C, TF32> r;
    gload(r, 0);
    sstore(r, 0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool more = kt + 1 < nk;
      if (more) gload(r, kt + 1);
      mma(kt & 1);
      if (more) sstore(r, (kt + 1) & 1, kt + 1);
      __syncthreads();
    }
    return;
  }
  Stage<C, TF32> r0, r1;
  gload(r0, 0);
  if (nk > 1) gload(r1, 1);
  sstore(r0, 0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    // stage kt is in LDS buffer 0, stage kt+1 is landing in r1
    if (kt + 2 < nk) gload(r0, kt + 2);
    mma(0);
    if (kt + 1 < nk) sstore(r1, 1, kt + 1);
    __syncthreads();
    if (kt + 1 >= nk) break;
    // stage kt+1 is in LDS buffer 1, stage kt+2 is landing in r0
    if (kt + 3 < nk) gload(r1, kt + 3);
    mma(1);
    if (kt + 2 < nk) sstore(r0, 0, kt + 2);
    __syncthreads();
  }
}

// threadIdx.x behind an empty asm: lane-dependent values derived from it are
// computed where they are used rather than hoisted by the compiler, where
// they would hold registers across the whole K loop.
__device__ __forceinline__ int tile_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS K loop (bf16 / int8 operands).
//
// gfx950's global_load_lds_dwordx4 writes lane l's 16 bytes to LDS at
// M0 + 16 l, so the loads need no staging registers and NSTAGE-1 stages of
// them can be in flight.  A stage holds 64 bytes of K for each of the BN + BM
// rows (row-major, 64 B per row).  Inside a row the four 16-byte chunks are
// stored XOR-swizzled, chunk c of row r at position c ^ ((r >> 2) & 3): the
// DMA lane that owns position p fetches chunk p ^ ((r >> 2) & 3).  gfx950's
// LDS serves a 16-byte read for 16 lanes per cycle across 64 banks (256 B);
// an MFMA operand read of chunk c by 16 consecutive rows then lands on 16
// distinct 16-byte slots of that 256-byte window (measured: without the
// swizzle every other LDS cycle was a bank conflict).
//
// The loads are issued from inline assembly, so the compiler does not insert
// its conservative waits on them; the loop waits itself (vmcnt), and each
// wait is followed by a workgroup barrier so that every wave's loads of the
// stage have landed before any wave reads it.  The barrier's "memory" clobber
// keeps the compiler from moving LDS reads across it.  M0 (the LDS address)
// is an input operand of the asm, so the compiler writes it and knows the
// asm leaves it unchanged.  An SALU write of M0 needs one wait state before
// an LDS-DMA load reads it; the compiler's hazard pass cannot see into the
// asm, so the asm starts with that wait state (s_nop 0).
typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_u8*)(void*)p;
}

__device__ __forceinline__ void dma16(uint32_t m0, const void* g) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(g), "{m0}"(m0) : "memory");
}

// The same load with the non-temporal hint (nt), for packed weight pieces
// that no other tile reads: whole lines streamed from HBM.  Measured on
// gfx950 with contiguous 1 KiB pieces, eight or four waves and a 3-stage
// ring: 6.9 TB/s against 6.1 TB/s without the hint.  Lines read again by
// other tiles then miss L2 (the prefill layer ran 23% slower with the hint on
// every packed load), and rows read as half lines are slower with it.
__device__ __forceinline__ void dma16_nt(uint32_t m0, const void* g) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" :: "v"(g), "{m0}"(m0) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" :: "n"(N) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
}

template <int NI>
__device__ __forceinline__ void wait_stage_nobar(int n_after) {
  switch (n_after) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<NI>(); break;
    case 2: wait_vm<2 * NI>(); break;
    case 3: wait_vm<3 * NI>(); break;
    default: wait_vm<4 * NI>(); break;
  }
}

template <int NI>
__device__ __forceinline__ void wait_stage(int n_after) {
  // wait until only n_after stages (NI loads each) of this wave are pending
  switch (n_after) {
    case 0: wait_vm_barrier<0>(); break;
    case 1: wait_vm_barrier<NI>(); break;
    case 2: wait_vm_barrier<2 * NI>(); break;
    case 3: wait_vm_barrier<3 * NI>(); break;
    default: wait_vm_barrier<4 * NI>(); break;
  }
}

// Bit of the packed-piece mask that asks for non-temporal weight loads: set
// when the tile is the only one that streams its weight slice (its expert
// has a single token block), so no other tile would find the lines in L2.
constexpr uint32_t kPkStream = 1u << 31;

//   NT_: the K loop can stream a sole reader's packed weights with the
//   non-temporal hint (a per-tile choice; configurations whose experts
//   nearly always span several blocks leave it out of the loop).
template <int BN_, int BM_, int NSTAGE_, int WN_ = 2, int WM_ = 2, int OCC_ = 1, bool NT_ = false>
struct DmaCfg {
  static constexpr int BN = BN_, BM = BM_, NSTAGE = NSTAGE_;
  static constexpr bool NT = NT_;
  static constexpr int OCC = OCC_;                           // workgroups per CU aimed for
  static constexpr int WN = WN_, WM = WM_, THREADS = 64 * WN * WM;
  static constexpr int ROWB = 64;                            // LDS bytes per row per stage
  static constexpr int RB = BN / WN / 32, CB = BM / WM / 32;
  static constexpr int NI = (BN + BM) / 16 / (WN * WM);      // DMA instructions per wave per stage
  static constexpr int kStage = (BN + BM) * ROWB;
  static constexpr int kBytes = NSTAGE * kStage;
  static_assert((BN + BM) % (16 * WN * WM) == 0 && NSTAGE >= 2 && NSTAGE <= 5, "dma tile shape");
  // vmcnt counts at most 63 outstanding loads per wave
  static_assert((NSTAGE - 1) * NI <= 63, "too many loads in flight for vmcnt");
};

// rowp[j]: global address of the start of this lane's j-th DMA row (local
// row (wave * NI + j) * 16 + lane / 4); every row is at least 16 bytes long.
// kbytes: bytes of K per row.  A partial last stage is handled by loading a
// valid chunk and zeroing it in LDS afterwards.
// Bit j of pk_mask (wave-uniform) marks rows held in the packed weight
// layout: there rowp[j] already points at this lane's 16 bytes of stage 0 and
// stage kt lies kt * kPackBlockBytes further (contiguous, pre-swizzled).
//   NCB: this wave's token column blocks that hold at least one valid row
//   (the valid rows of a tile come first); the others are neither read from
//   LDS nor multiplied.  Every wave still issues its loads and meets every
//   barrier.
template <class C, int KIND, int NCB>
__device__ __forceinline__ void mainloop_dma(uint8_t* smem, const uint8_t* const (&rowp)[C::NI],
                                             uint32_t pk_mask, int64_t kbytes,
                                             const int (&wrow)[C::RB], int tcol0,
                                             typename Mma<KIND>::acc_t (&acc)[C::RB][C::CB]) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const uint32_t sbase = lds_addr(smem);
  const int chunk_pos = lane & 3;
  const int nk = (int)((kbytes + C::ROWB - 1) / C::ROWB);

  auto issue = [&](int kt) {
    const uint32_t st = sbase + (uint32_t)((kt % C::NSTAGE) * C::kStage);
    const int64_t koff = (int64_t)kt * C::ROWB;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
      const int row = (wave * C::NI + j) * 16 + (lane >> 2);
      const int c = chunk_pos ^ ((row >> 2) & 3);            // chunk this lane fetches
      const int64_t off = ((pk_mask >> j) & 1u)
                              ? (int64_t)kt * kPackBlockBytes
                              : (koff + c * 16 < kbytes ? koff + c * 16 : 0);   // past K: row start
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(st + (uint32_t)((wave * C::NI + j) * 1024));
      if (C::NT && (pk_mask & kPkStream) && ((pk_mask >> j) & 1u)) dma16_nt(m0, rowp[j] + off);
      else dma16(m0, rowp[j] + off);
    }
  };
  // zero the chunks of a partial stage that lie past K (after its loads landed)
  auto zero_tail = [&](int kt) {
    uint8_t* st = smem + (kt % C::NSTAGE) * C::kStage;
    const int64_t koff = (int64_t)kt * C::ROWB;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
      const int row = (wave * C::NI + j) * 16 + (lane >> 2);
      const int c = chunk_pos ^ ((row >> 2) & 3);
      if (koff + c * 16 >= kbytes)
        *reinterpret_cast<u32x4_t*>(st + (wave * C::NI + j) * 1024 + lane * 16) =
            u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  // MFMA operand fragments are double-buffered in registers: the LDS reads
  // of the next k-step (32 elements of K) are in flight while the MFMAs of
  // the current one run; the first k-step of the next stage is read right
  // after the barrier that publishes it.
  const int swz = ((lane & 31) >> 2) & 3;
  auto load_frags = [&](int kt, int ks, u32x4_t (&af)[C::RB], u32x4_t (&bf)[C::CB]) {
    const uint8_t* st = smem + (kt % C::NSTAGE) * C::kStage + (lane & 31) * C::ROWB;
    const int pos = ((ks * 2 + (lane >> 5)) ^ swz) * 16;
    if constexpr (NCB > 0) {
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
        af[rb] = *reinterpret_cast<const u32x4_t*>(st + wrow[rb] * C::ROWB + pos);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      bf[cb] = *reinterpret_cast<const u32x4_t*>(st + (C::BN + tcol0 + cb * 32) * C::ROWB + pos);
  };
  auto mfmas = [&](const u32x4_t (&af)[C::RB], const u32x4_t (&bf)[C::CB]) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) acc[rb][cb] = Mma<KIND>::run(af[rb], bf[cb], acc[rb][cb]);
  };
  const bool partial = (kbytes % C::ROWB) != 0;
  // Publish stage s: this wave's loads of it have landed (n_after later
  // stages may still be pending), then all waves meet at the barrier.
  auto publish = [&](int s, int n_after) {
    if (partial && s == nk - 1) {
      wait_stage_nobar<C::NI>(0);
      zero_tail(s);
      __syncthreads();
    } else {
      wait_stage<C::NI>(n_after);
    }
  };

  // Stage s goes to LDS buffer s % NSTAGE; all NSTAGE buffers start loading.
  const int pre = nk < C::NSTAGE ? nk : C::NSTAGE;
  for (int kt = 0; kt < pre; ++kt) issue(kt);
  u32x4_t a0[C::RB], b0[C::CB], a1[C::RB], b1[C::CB];
  publish(0, pre - 1);
  load_frags(0, 0, a0, b0);
  for (int kt = 0; kt < nk; ++kt) {
    load_frags(kt, 1, a1, b1);
    mfmas(a0, b0);
    if (kt + 1 < nk) {
      const int last = (kt + C::NSTAGE - 1 < nk - 1) ? kt + C::NSTAGE - 1 : nk - 1;
      publish(kt + 1, last - (kt + 1));
      // every wave has finished reading stage kt: refill its buffer
      if (kt + C::NSTAGE < nk) issue(kt + C::NSTAGE);
      load_frags(kt + 1, 0, a0, b0);
    }
    mfmas(a1, b1);
  }
}

// Runs the K loop specialised for this wave's number of live column blocks
// (wave-uniform), so the loop itself has no per-block branches.
template <class C, int KIND>
__device__ __forceinline__ void mainloop_dma_live(uint8_t* smem, const uint8_t* const (&rowp)[C::NI],
                                                  uint32_t pk_mask, int64_t kbytes,
                                                  const int (&wrow)[C::RB], int tcol0,
                                                  int valid_rows,
                                                  typename Mma<KIND>::acc_t (&acc)[C::RB][C::CB]) {
  int ncb = (valid_rows - tcol0 + 31) / 32;
  ncb = __builtin_amdgcn_readfirstlane(ncb < 0 ? 0 : (ncb > C::CB ? C::CB : ncb));
  pk_mask = __builtin_amdgcn_readfirstlane(pk_mask);
  if constexpr (C::CB >= 4) {
    if (ncb == 4) return mainloop_dma<C, KIND, 4>(smem, rowp, pk_mask, kbytes, wrow, tcol0, acc);
    if (ncb == 3) return mainloop_dma<C, KIND, 3>(smem, rowp, pk_mask, kbytes, wrow, tcol0, acc);
  }
  if constexpr (C::CB >= 2) {
    if (ncb == 2) return mainloop_dma<C, KIND, 2>(smem, rowp, pk_mask, kbytes, wrow, tcol0, acc);
  }
  if (ncb == 1) return mainloop_dma<C, KIND, 1>(smem, rowp, pk_mask, kbytes, wrow, tcol0, acc);
  mainloop_dma<C, KIND, 0>(smem, rowp, pk_mask, kbytes, wrow, tcol0, acc);
}

// ---------------------------------------------------------------------------
// Weight-row sources of a thread: local rows lrow + STEP i, i < WR; rows of
// the second half (i >= WR/2) come from w[1].  `first` is the global row of
// local row lrow in the first half, `second` that of the second half, and
// `limit` bounds both halves' rows counted from `first` / `second`.
template <class C>
__device__ __forceinline__ void weight_src(Src<C>& src, const uint8_t* base, int64_t row_bytes,
                                           int64_t first, int64_t second, int64_t limit0,
                                           int64_t limit1) {
  constexpr int HALF = C::WR / 2;
  src.wstep = (int64_t)C::STEP * row_bytes;
  const int64_t n0 = limit0 > 0 ? (limit0 + C::STEP - 1) / C::STEP : 0;
  const int64_t n1 = limit1 > 0 ? (limit1 + C::STEP - 1) / C::STEP : 0;
  const int last0 = (int)(n0 < HALF ? n0 : HALF) - 1;
  const int last1 = (int)(n1 < HALF ? n1 : HALF) - 1;
  src.w[0] = last0 >= 0 ? base + first * row_bytes : base;
  src.w[1] = last1 >= 0 ? base + second * row_bytes : base;
  src.wlast[0] = last0;
  src.wlast[1] = last1;
}

// Fused-MoE grouped GEMM (bf16 weights, MFMA bf16 -> f32).
//   EPI 0: C = acc;  EPI 1: C[:, j] = silu(acc_gate_j) * acc_up_j.
//   TF32: tokens are float32 rows (rounded to bf16 on the way to LDS; these
//   tiles use the register-staged loop, the others the direct-to-LDS loop).

// Tile of the sorted list handled by this workgroup; false if none.
struct MoeTile {
  int blk, nt, e;
  int64_t s0, c0;
  int solo = 0;   // the expert has one token block: no other tile reads this weight slice
};

// Output tiles along N.
template <int BN, int EPI>
__device__ __forceinline__ int moe_ntiles(const MoeGemmArgs& a) {
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int64_t ncols = EPI ? BN / 2 : BN;            // output columns per tile
  return (int)((Nout + ncols - 1) / ncols);
}

// Tile of logical index L, 0 <= L < nblk * ntile.  Block-major numbering
// (L = blk * ntile + nt) gives each expert one contiguous range of
// m_e * ntile tiles.  Inside that range the tiles are renumbered
// n-tile-major (L = base + nt * m_e + mb), so the m_e tiles that read the
// same weight slice are neighbours: they are dispatched together and stream
// that slice through L2 once.  The workgroup finds its expert's block range
// from one read of expert_ids around its block-major block (a window of
// blockDim.x blocks).  Experts longer than half the window keep block-major
// order; that choice depends only on the expert, so every workgroup of an
// expert uses the same numbering and the mapping stays a bijection.  Uses
// two barriers; s_win: 3 ints of LDS.
template <int BN, int BM, int EPI>
__device__ __forceinline__ bool moe_tile_at(const MoeGemmArgs& a, int L, int nblk, MoeTile& t,
                                            int* s_win) {
  const int64_t ncols = EPI ? BN / 2 : BN;
  const int ntile = moe_ntiles<BN, EPI>(a);
  const int bm = L / ntile;                           // block-major block
  const int half = (int)blockDim.x / 2;
  const int idx = bm - half + (int)tile_tid();       // window [bm - half, bm + half)
  const int v = (idx >= 0 && idx < nblk) ? a.expert_ids[idx] : -2;
  if (tile_tid() == 0) { s_win[1] = INT32_MAX; s_win[2] = -1; }
  if (idx == bm) s_win[0] = v;
  __syncthreads();
  const int e = s_win[0];
  if (v == e) { atomicMin(&s_win[1], idx); atomicMax(&s_win[2], idx); }
  __syncthreads();
  const int first = s_win[1], last = s_win[2];
  const bool first_exact = first > bm - half || first == 0;
  const bool last_exact = last < bm + half - 1 || last == nblk - 1;
  const int m_e = last - first + 1;
  if (e >= 0 && first_exact && last_exact && m_e <= half - 1) {
    const int local = L - first * ntile;
    t.nt = local / m_e;
    t.blk = first + local % m_e;
  } else {
    t.blk = bm;
    t.nt = L % ntile;
  }
  t.e = e;
  t.s0 = (int64_t)t.blk * BM;
  t.c0 = (int64_t)t.nt * ncols;
  t.solo = e >= 0 && first_exact && last_exact && m_e == 1;
  return t.e >= 0;
}

// Tile of this workgroup in a grid of one workgroup per tile; false if none.
// Logical tile L is workgroup L, so consecutive tiles (an expert's n-tiles)
// go to consecutive XCDs and every XCD streams a share of every expert's
// weights.  (Measured on the decode layers against giving each XCD one
// contiguous run of tiles: T = 16 1404 against 1422 us, T = 64 2818 against
// 2891 us.)
template <int BN, int BM, int EPI>
__device__ __forceinline__ bool moe_tile(const MoeGemmArgs& a, MoeTile& t, int* s_win) {
  const int nblk = *a.total / BM;
  const int live = nblk * moe_ntiles<BN, EPI>(a);
  if ((int)blockIdx.x >= live) return false;
  return moe_tile_at<BN, BM, EPI>(a, (int)blockIdx.x, nblk, t, s_win);
}

// Local weight row of tile row r (0 <= r < BN) -> global row of expert e,
// or -1 past the matrix.  With the SiLU epilogue rows [0, BN/2) are gate
// rows c0 + r and rows [BN/2, BN) the up rows of the same columns.
template <int BN, int EPI>
__device__ __forceinline__ int64_t moe_weight_row(const MoeGemmArgs& a, int64_t c0, int r) {
  if (EPI) {
    const int64_t Nout = a.N / 2;
    const int64_t hcol = c0 + (r < BN / 2 ? r : r - BN / 2);
    if (hcol >= Nout) return -1;
    return r < BN / 2 ? hcol : Nout + hcol;
  }
  const int64_t n = c0 + r;
  return n < a.N ? n : -1;
}

// First local weight row of each of this wave's 32-row blocks; with the SiLU
// epilogue block rb < RB/2 holds gate rows, block rb + RB/2 the matching up rows.
template <int BN, int WN, int RB, int EPI>
__device__ __forceinline__ void wave_rows(int wn, int (&wrow)[RB]) {
  constexpr int WROWS = BN / WN;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    wrow[rb] = EPI ? ((rb < RB / 2) ? wn * (WROWS / 2) + rb * 32
                                    : BN / 2 + wn * (WROWS / 2) + (rb - RB / 2) * 32)
                   : wn * WROWS + rb * 32;
}

// Epilogue.  32x32 MFMA output: lane holds token column (lane & 31) and, for
// g = 0..3, rows 8 g + 4 (lane >> 5) + [0, 4) of its 32-row block.
// fp32 values of accumulator entries 4g .. 4g+3: the sums themselves (bf16
// MFMA), or the exact int32 sums times the row scale and four channel
// scales (int8 MFMA).
__device__ __forceinline__ f32x4_t acc4(const f32x16_t& a, int g, float, const f32x4_t&) {
  return f32x4_t{a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
}
__device__ __forceinline__ f32x4_t acc4(const i32x16_t& a, int g, float as, const f32x4_t& bs) {
  return f32x4_t{(float)a[4 * g] * as * bs[0], (float)a[4 * g + 1] * as * bs[1],
                 (float)a[4 * g + 2] * as * bs[2], (float)a[4 * g + 3] * as * bs[3]};
}
// Outputs 4g .. 4g+3 of a row without the SiLU epilogue (the down GEMM):
// the bf16 MFMA sums times the row's routing weight w, or the exact int32
// sums times the row factor rf = a_scales[row] * w (one product per row),
// then the four channel scales: two multiplies per output, all epilogues
// of this GEMM in the same order.
__device__ __forceinline__ f32x4_t row4(const f32x16_t& a, int g, float w, const f32x4_t&) {
  return f32x4_t{a[4 * g] * w, a[4 * g + 1] * w, a[4 * g + 2] * w, a[4 * g + 3] * w};
}
__device__ __forceinline__ f32x4_t row4(const i32x16_t& a, int g, float rf, const f32x4_t& bs) {
  return f32x4_t{(float)a[4 * g] * rf * bs[0], (float)a[4 * g + 1] * rf * bs[1],
                 (float)a[4 * g + 2] * rf * bs[2], (float)a[4 * g + 3] * rf * bs[3]};
}

// Epilogue.  32x32 MFMA output: lane holds token column (lane & 31) and, for
// g = 0..3, rows 8 g + 4 (lane >> 5) + [0, 4) of its 32-row block.
template <int RB, int CB, int EPI, int CDT, int KIND>
__device__ __forceinline__ void moe_epilogue(const MoeGemmArgs& a, const MoeTile& t,
                                             const int* rowinfo, const int (&wrow)[RB], int tcol0,
                                             const typename Mma<KIND>::acc_t (&acc)[RB][CB]) {
  const int lane = tile_tid() & 63;
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  uint8_t* Cb = reinterpret_cast<uint8_t*>(a.C);
  constexpr int ce = ElemBytes<CDT>::value;
  const int rsub = 4 * (lane >> 5);
  const float* bsc = KIND ? a.b_scales + (int64_t)t.e * a.N : nullptr;
  const f32x4_t one4 = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int trow = tcol0 + cb * 32 + (lane & 31);
    const int p = rowinfo[trow];
    if (p < 0 || p >= a.num_valid) continue;
    const int64_t crow = (a.c_rows == 0) ? (int64_t)p : t.s0 + trow;
    const float w = a.topk_weights ? a.topk_weights[p] : 1.0f;
    float as = 1.0f;
    if constexpr (KIND != 0)
      as = a.a_scales[a.a_rows == 0 ? (int64_t)(p / a.a_row_div) : t.s0 + trow];
    uint8_t* rowp = Cb + crow * a.ldc * ce;
    if (EPI) {
#pragma unroll
      for (int j = 0; j < RB / 2; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = t.c0 + wrow[j] + 8 * g + rsub;
          if (col < Nout) {
            f32x4_t sg = one4, su = one4;
            if constexpr (KIND != 0) {
              sg = *reinterpret_cast<const f32x4_t*>(bsc + col);
              su = *reinterpret_cast<const f32x4_t*>(bsc + Nout + col);
            }
            const f32x4_t gt = acc4(acc[j][cb], g, as, sg);
            const f32x4_t up = acc4(acc[j + RB / 2][cb], g, as, su);
            store4<CDT>(rowp + col * ce, silu_f32(gt[0]) * up[0] * w, silu_f32(gt[1]) * up[1] * w,
                        silu_f32(gt[2]) * up[2] * w, silu_f32(gt[3]) * up[3] * w);
          }
        }
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t col = t.c0 + wrow[rb] + 8 * g + rsub;
          if (col < a.N) {
            f32x4_t sc = one4;
            if constexpr (KIND != 0) sc = *reinterpret_cast<const f32x4_t*>(bsc + col);
            const f32x4_t v = row4(acc[rb][cb], g, KIND ? as * w : w, sc);
            store4<CDT>(rowp + col * ce, v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }
}

template <int BM>
__device__ __forceinline__ void load_rowinfo(const MoeGemmArgs& a, const MoeTile& t, int* rowinfo) {
  for (int r = tile_tid(); r < BM; r += blockDim.x) {
    const int p = a.sorted_ids[t.s0 + r];
    rowinfo[r] = (p >= 0 && p < a.num_valid) ? p : -1;
  }
  __syncthreads();
}

// 1 + the last tile row holding a valid pair (0 if none); wave-uniform.
// rowinfo: the tile's entries, -1 or a raw sorted id (>= num_valid = placeholder).
template <int BM>
__device__ __forceinline__ int live_rows(const int* rowinfo, int64_t num_valid) {
  const int lane = tile_tid() & 63;
  uint32_t last = 0;
#pragma unroll
  for (int r = lane; r < BM; r += 64) {
    const int p = rowinfo[r];
    if (p >= 0 && p < num_valid) last = (uint32_t)(r + 1);
  }
  return (int)wave_max_u32(last);
}

// A row feeding tile token row r; placeholder rows read the tile's first row
// (valid whenever row 0 is), which only reaches masked outputs.  rowinfo
// entries are -1 or raw sorted ids (>= num_valid = placeholder).
__device__ __forceinline__ int moe_token_row(const MoeGemmArgs& a, const MoeTile& t,
                                             const int* rowinfo, int r) {
  const int p = rowinfo[r];
  if (p < 0 || p >= a.num_valid) {
    const int p0 = rowinfo[0];
    return (p0 < 0 || p0 >= a.num_valid) ? 0 : (a.a_rows == 0 ? p0 / a.a_row_div : (int)t.s0);
  }
  return a.a_rows == 0 ? p / a.a_row_div : (int)(t.s0 + r);
}

// Register-staged variant (float32 tokens).
template <class C, int EPI, int CDT>
__global__ void __launch_bounds__(C::THREADS) moe_gemm_tile_kernel(MoeGemmArgs a) {
  typedef C S;
  constexpr int BN = C::BN, BM = C::BM;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int rowinfo[BM];
  MoeTile t;
  __shared__ int s_win[3];
  if (!moe_tile<BN, BM, EPI>(a, t, s_win)) return;
  load_rowinfo<BM>(a, t, rowinfo);

  const int tid = tile_tid(), wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;
  const int lrow = tid >> 3;
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int64_t wrow_bytes = a.K * 2;
  const uint8_t* Bw = reinterpret_cast<const uint8_t*>(a.B) + (int64_t)t.e * a.N * wrow_bytes;
  Src<C> src;
  if (EPI)   // first half: gate rows c0 + ..., second half: the matching up rows
    weight_src<C>(src, Bw, wrow_bytes, t.c0 + lrow, Nout + t.c0 + lrow, Nout - t.c0 - lrow,
                  Nout - t.c0 - lrow);
  else
    weight_src<C>(src, Bw, wrow_bytes, t.c0 + lrow, t.c0 + BN / 2 + lrow, a.N - t.c0 - lrow,
                  a.N - t.c0 - BN / 2 - lrow);
  src.abase = reinterpret_cast<const uint8_t*>(a.A);
  src.arow_bytes = a.lda * 4;
#pragma unroll
  for (int i = 0; i < S::TR; ++i) src.trow[i] = moe_token_row(a, t, rowinfo, lrow + S::STEP * i);

  int wrow[S::RB];
  wave_rows<BN, C::WN, S::RB, EPI>(wn, wrow);
  const int tcol0 = wm * (BM / C::WM);
  f32x16_t acc[S::RB][S::CB];
#pragma unroll
  for (int rb = 0; rb < S::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < S::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0.0f;
  mainloop<C, 0, true>(smem, src, wrow_bytes, wrow, tcol0, acc);
  moe_epilogue<S::RB, S::CB, EPI, CDT, 0>(a, t, rowinfo, wrow, tcol0, acc);
}

// SiLU epilogue with bf16 output that stages the tile in LDS and writes
// whole 256-byte row segments (written straight from the MFMA layout each
// store instruction would touch 32 rows with 16 bytes each).  Reuses the K
// ring, which every wave has finished reading at the first barrier.  wr / ar: this thread's
// row weight and (int8) row scale (threads < BM), read before the K loop.
template <class C, int KIND>
__device__ __forceinline__ void silu_epilogue_staged(const MoeGemmArgs& a, const MoeTile& t,
                                                     const int* rowinfo,
                                                     const int (&wrow)[C::RB], int tcol0,
                                                     const typename Mma<KIND>::acc_t (&acc)[C::RB][C::CB],
                                                     uint8_t* smem, float wr, float ar) {
  constexpr int RB = C::RB, CB = C::CB, BM = C::BM, HC = C::BN / 2;   // BM rows x HC columns
  constexpr int PITCH = HC * 2 + 16;          // LDS bytes per token row
  constexpr int LPR = HC * 2 / 16;            // lanes per row in the store phase
  constexpr int RPP = C::THREADS / LPR;       // rows per store pass
  static_assert(BM * PITCH + 2 * BM * 4 <= C::kBytes && C::THREADS % LPR == 0 && BM % RPP == 0 &&
                    BM <= C::THREADS,
                "staged epilogue shape");
  float* s_w = reinterpret_cast<float*>(smem + BM * PITCH);
  float* s_a = s_w + BM;
  const int tid = tile_tid(), lane = tid & 63;
  const int rsub = 4 * (lane >> 5);
  const int64_t Nout = a.N / 2;
  const float* bsc = KIND ? a.b_scales + (int64_t)t.e * a.N : nullptr;
  const f32x4_t one4 = {1.0f, 1.0f, 1.0f, 1.0f};
  __syncthreads();                            // every wave has left the K ring
  if (tid < BM) { s_w[tid] = wr; s_a[tid] = ar; }
  __syncthreads();
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int trow = tcol0 + cb * 32 + (lane & 31);
    const float w = s_w[trow], as = s_a[trow];
    uint8_t* dst = smem + trow * PITCH;
#pragma unroll
    for (int j = 0; j < RB / 2; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wrow[j] + 8 * g + rsub;
        f32x4_t sg = one4, su = one4;
        if constexpr (KIND != 0) {
          const int64_t gc = t.c0 + col < Nout ? t.c0 + col : 0;   // past N: never stored
          sg = *reinterpret_cast<const f32x4_t*>(bsc + gc);
          su = *reinterpret_cast<const f32x4_t*>(bsc + Nout + gc);
        }
        const f32x4_t gt = acc4(acc[j][cb], g, as, sg);
        const f32x4_t up = acc4(acc[j + RB / 2][cb], g, as, su);
        const uint2 v = make_uint2(
            pack_bf16x2(silu_f32(gt[0]) * up[0] * w, silu_f32(gt[1]) * up[1] * w),
            pack_bf16x2(silu_f32(gt[2]) * up[2] * w, silu_f32(gt[3]) * up[3] * w));
        *reinterpret_cast<uint2*>(dst + col * 2) = v;
      }
    }
  }
  __syncthreads();
  uint8_t* Cb = reinterpret_cast<uint8_t*>(a.C);
  const int ch = tid % LPR;
  const int64_t col = t.c0 + ch * 8;          // 8 columns; Nout is a multiple of 8
#pragma unroll
  for (int r0 = 0; r0 < BM; r0 += RPP) {
    const int r = r0 + tid / LPR;
    const int p = rowinfo[r];
    if (p < 0 || p >= a.num_valid || col >= Nout) continue;
    const int64_t crow = (a.c_rows == 0) ? (int64_t)p : t.s0 + r;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + r * PITCH + ch * 16);
    *reinterpret_cast<u32x4_t*>(Cb + (crow * a.ldc + col) * 2) = v;
  }
}

// Plain epilogue (bf16 or f16 output, bf16 MFMA) through LDS: the tile is
// written into the drained K ring in [token row][column] order, then each
// output row's BN columns go out as whole 16-byte pieces, 32 lanes per row.
// Straight from the MFMA layout each store instruction would cover 32 rows
// with 16 bytes each.  wr: this thread's row weight (threads < BM), read
// before the K loop.
template <class C, int CDT, int KIND>
__device__ __forceinline__ void plain_epilogue_staged(const MoeGemmArgs& a, const MoeTile& t,
                                                      const int* rowinfo,
                                                      const int (&wrow)[C::RB], int tcol0,
                                                      const typename Mma<KIND>::acc_t (&acc)[C::RB][C::CB],
                                                      uint8_t* smem, float wr, float ar) {
  constexpr int RB = C::RB, CB = C::CB, BM = C::BM, BN = C::BN;
  constexpr int PITCH = BN * 2 + 16;          // LDS bytes per token row
  constexpr int LPR = BN * 2 / 16;            // lanes per row in the store phase
  constexpr int RPP = C::THREADS / LPR;       // rows per store pass
  static_assert(BM * PITCH + 2 * BM * 4 <= C::kBytes && C::THREADS % LPR == 0 && BM % RPP == 0 &&
                    BM <= C::THREADS && (CDT == 1 || CDT == 2),
                "staged epilogue shape");
  float* s_w = reinterpret_cast<float*>(smem + BM * PITCH);
  float* s_a = s_w + BM;
  const int tid = tile_tid(), lane = tid & 63;
  const int rsub = 4 * (lane >> 5);
  const float* bsc = KIND ? a.b_scales + (int64_t)t.e * a.N : nullptr;
  const f32x4_t one4 = {1.0f, 1.0f, 1.0f, 1.0f};
  __syncthreads();                            // every wave has left the K ring
  if (tid < BM) { s_w[tid] = wr; s_a[tid] = ar; }
  __syncthreads();
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int trow = tcol0 + cb * 32 + (lane & 31);
    const float w = s_w[trow], as = s_a[trow];
    uint8_t* dst = smem + trow * PITCH;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t sc = one4;
        if constexpr (KIND != 0) {
          const int64_t gc = t.c0 + wrow[rb] + 8 * g + rsub;
          sc = *reinterpret_cast<const f32x4_t*>(bsc + (gc < a.N ? gc : 0));   // past N: never stored
        }
        const f32x4_t v = row4(acc[rb][cb], g, KIND ? as * w : w, sc);
        const float a0 = v[0], a1 = v[1], a2 = v[2], a3 = v[3];
        const uint2 o = CDT == 1 ? make_uint2(pack_bf16x2(a0, a1), pack_bf16x2(a2, a3))
                                 : make_uint2(pack_f16x2(a0, a1), pack_f16x2(a2, a3));
        *reinterpret_cast<uint2*>(dst + (wrow[rb] + 8 * g + rsub) * 2) = o;
      }
    }
  }
  __syncthreads();
  uint8_t* Cb = reinterpret_cast<uint8_t*>(a.C);
  const int ch = tid % LPR;
  const int64_t col = t.c0 + ch * 8;          // 8 columns; N is a multiple of 16
#pragma unroll
  for (int r0 = 0; r0 < BM; r0 += RPP) {
    const int r = r0 + tid / LPR;
    const int p = rowinfo[r];
    if (p < 0 || p >= a.num_valid || col >= a.N) continue;
    const int64_t crow = (a.c_rows == 0) ? (int64_t)p : t.s0 + r;
    *reinterpret_cast<u32x4_t*>(Cb + (crow * a.ldc + col) * 2) =
        *reinterpret_cast<const u32x4_t*>(smem + r * PITCH + ch * 16);
  }
}

// One tile with the direct-to-LDS loop (rowinfo already loaded): operand
// addresses, K loop, epilogue.
template <class C, int EPI, int CDT, int KIND>
__device__ __forceinline__ void run_dma_tile(const MoeGemmArgs& a, const MoeTile& t, uint8_t* smem,
                                             const int* rowinfo) {
  constexpr int BN = C::BN, BM = C::BM;

  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;
  constexpr int eb = KIND ? 1 : 2;                 // operand element bytes
  const int64_t wrow_bytes = a.K * eb;
  const uint8_t* Bw = reinterpret_cast<const uint8_t*>(a.B) + (int64_t)t.e * a.N * wrow_bytes;
  const uint8_t* Ab = reinterpret_cast<const uint8_t*>(a.A);
  const int64_t arow_bytes = a.lda * eb;
  // packed weights: a tile of BN rows is SUB = BN / kPackRows consecutive
  // packed tiles.  The LDS rows keep the plain order (with the SiLU epilogue
  // the BN/2 gate rows, then the BN/2 up rows), so piece q of the stage
  // (LDS rows 16q .. 16q+15) comes from packed tile nt * SUB + s, rows pr ..:
  //   SiLU:  gate row R < BN/2      -> s = R / 128, pr = R % 128;
  //          up row R >= BN/2       -> s = (R - BN/2) / 128, pr = 128 + (R - BN/2) % 128;
  //   plain: s = R / 256, pr = R % 256.
  // A packed tile past the matrix (its rows are never stored) reads the
  // tile's first packed tile instead.  Row and packed row agree mod 16, so
  // the pre-swizzled chunk order is the one the LDS rows expect.
  constexpr int SUB = BN / kPackRows;
  const int64_t kst = packed_kstages(a.K, eb);
  const int64_t ptiles = packed_tiles(a.N, EPI);
  const uint8_t* Bp = reinterpret_cast<const uint8_t*>(a.B) +
                      ((int64_t)t.e * ptiles + (int64_t)t.nt * SUB) * kst * kPackBlockBytes;
  const uint8_t* rowp[C::NI];
  uint32_t pk_mask = 0;
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int q = wave * C::NI + j;            // 1 KiB piece of the stage: rows 16q .. 16q+15
    const int r = q * 16 + (lane >> 2);
    if (q < BN / 16) {
      if (a.b_packed) {
        const int R = q * 16;
        int sub, pr;
        if (EPI) {
          const int Rg = R < BN / 2 ? R : R - BN / 2;
          sub = Rg / (kPackRows / 2);
          pr = (R < BN / 2 ? 0 : kPackRows / 2) + Rg % (kPackRows / 2);
        } else {
          sub = R / kPackRows;
          pr = R % kPackRows;
        }
        if ((int64_t)t.nt * SUB + sub >= ptiles) sub = 0;
        rowp[j] = Bp + (int64_t)sub * kst * kPackBlockBytes + pr * 64 + lane * 16;
        pk_mask |= 1u << j;
      } else {
        const int64_t g = moe_weight_row<BN, EPI>(a, t.c0, r);
        rowp[j] = Bw + (g < 0 ? 0 : g) * wrow_bytes;      // past the matrix: row 0
      }
    } else {
      rowp[j] = Ab + (int64_t)moe_token_row(a, t, rowinfo, r - BN) * arow_bytes;
    }
  }
  if (t.solo && pk_mask) pk_mask |= kPkStream;
  int wrow[C::RB];
  wave_rows<BN, C::WN, C::RB, EPI>(wn, wrow);
  const int tcol0 = wm * (BM / C::WM);
  typename Mma<KIND>::acc_t acc[C::RB][C::CB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0;
  // 16-bit output goes out through LDS when the tile fits the ring (SiLU:
  // bf16 output only)
  constexpr bool kStagedPlain = EPI == 0 && (CDT == 1 || CDT == 2) &&
                                BM * (BN * 2 + 16) + 2 * BM * 4 <= C::kBytes && BM <= C::THREADS;
  constexpr bool kStagedSilu = EPI == 1 && CDT == 1 &&
                               BM * (BN + 16) + 2 * BM * 4 <= C::kBytes && BM <= C::THREADS;
  // this thread's row weight and (int8) row scale, read while the K loop runs
  float wr = 1.0f, ar = 1.0f;
  if constexpr (kStagedPlain || kStagedSilu) {
    if (tid < BM) {
      const int p = rowinfo[tid];
      if (p >= 0 && p < a.num_valid) {
        if (a.topk_weights) wr = a.topk_weights[p];
        if constexpr (KIND != 0)
          ar = a.a_scales[a.a_rows == 0 ? (int64_t)(p / a.a_row_div) : t.s0 + tid];
      }
    }
  }
  mainloop_dma_live<C, KIND>(smem, rowp, pk_mask, wrow_bytes, wrow, tcol0,
                             live_rows<BM>(rowinfo, a.num_valid), acc);
  if constexpr (kStagedSilu) {
    silu_epilogue_staged<C, KIND>(a, t, rowinfo, wrow, tcol0, acc, smem, wr, ar);
  } else if constexpr (kStagedPlain) {
    plain_epilogue_staged<C, CDT, KIND>(a, t, rowinfo, wrow, tcol0, acc, smem, wr, ar);
  } else {
    moe_epilogue<C::RB, C::CB, EPI, CDT, KIND>(a, t, rowinfo, wrow, tcol0, acc);
  }
}

// Direct-to-LDS variant (bf16 tokens), one workgroup per tile.
//   KIND 0: bf16 tokens and weights; KIND 1: int8 tokens and weights with
//   per-row and per-channel scales applied in the epilogue.
template <class C, int EPI, int CDT, int KIND>
__global__ void __launch_bounds__(C::THREADS, C::OCC * C::THREADS / 256)
moe_gemm_dma_kernel(MoeGemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int rowinfo[C::BM];
  MoeTile t;
  __shared__ int s_win[3];
  if (!moe_tile<C::BN, C::BM, EPI>(a, t, s_win)) return;
  load_rowinfo<C::BM>(a, t, rowinfo);   // one global round trip, then LDS
  run_dma_tile<C, EPI, CDT, KIND>(a, t, smem, rowinfo);
}

// ---------------------------------------------------------------------------
// INT8 GMM: rows [off[e], off[e+1]) of X use W[e]; fp16 output.
#ifndef MOE_GMM_NSTAGE
#define MOE_GMM_BM 128
#define MOE_GMM_NSTAGE 3
#define MOE_GMM_OCC 2
#define MOE_GMM_WN 4
#define MOE_GMM_WM 2
#endif
typedef DmaCfg<256, MOE_GMM_BM, MOE_GMM_NSTAGE, MOE_GMM_WN, MOE_GMM_WM, MOE_GMM_OCC, true> GmmCfg;
static_assert(GmmCfg::BN == kPackRows, "packed int8 weights are cut into tiles of BN rows");

typedef i32x16_t GmmAcc[GmmCfg::RB][GmmCfg::CB];

__device__ __forceinline__ int gmm_row_of(const GmmI8Args& a, int e) {
  const int v = a.offsets[e], M = (int)a.M;
  return v < 0 ? 0 : (v > M ? M : v);
}

// Order of the GMM's tiles.  A weight slice (expert e, n-tile nt) has one
// tile per m-tile of e; those run back to back on one XCD, so the slice is
// fetched once into that XCD's L2.  Slices are dealt to the 8 XCDs
// round-robin in the order: experts by rows, most first (ties by id), then
// n-tiles, so every XCD streams an even share of every expert's weights and
// runs its slices in that order.  Workgroup id i is placed on XCD i % 8
// (slot i / 8 of that XCD's sequence): each XCD starts with its share of the
// largest experts, and the tiles left for the slots that free up first are
// those of the smallest.
struct GmmOrder {
  int prefix[kMaxGmmExperts + 1];   // this XCD's tiles before sorted position p
  uint16_t order[kMaxGmmExperts];   // expert at sorted position p
};

// n-tiles nt in [0, ntile) with (p * ntile + nt) % 8 == xcd: the first one and
// how many.
__device__ __forceinline__ int gmm_first_nt(int p, int ntile, int xcd) {
  const int base = ((p % kNumXcd) * (ntile % kNumXcd)) % kNumXcd;
  return (xcd - base + kNumXcd) % kNumXcd;
}
__device__ __forceinline__ int gmm_units_on(int p, int ntile, int xcd) {
  const int nt0 = gmm_first_nt(p, ntile, xcd);
  return nt0 < ntile ? (ntile - 1 - nt0) / kNumXcd + 1 : 0;
}

// Builds o for this workgroup's XCD.  work: at least THREADS + E + 4 ints of
// LDS that are free until the K loop (rows per expert, then the scan).
// Every thread takes part (barriers).
__device__ __forceinline__ void gmm_build_order(const GmmI8Args& a, int ntile, int xcd,
                                                GmmOrder& o, int* work) {
  constexpr int BM = GmmCfg::BM, NT = GmmCfg::THREADS;
  constexpr int PER = (kMaxGmmExperts + NT - 1) / NT;   // sorted positions per thread
  const int tid = tile_tid(), E = a.E, E4 = (E + 3) & ~3;
  int* rows = work;                 // [E4]; -1 past E sorts after every expert
  int* scan_buf = work + E4;        // [NT]
  for (int e = tid; e < E4; e += NT) {
    int r = -1;
    if (e < E) {
      const int lo = gmm_row_of(a, e), hi = gmm_row_of(a, e + 1);
      r = hi > lo ? hi - lo : 0;
    }
    rows[e] = r;
  }
  __syncthreads();
  // sorted position of e: experts with more rows, or as many rows and a
  // smaller id, come first
  for (int e = tid; e < E; e += NT) {
    const int re = rows[e];
    int pos = 0;
    for (int f = 0; f < E4; f += 4) {
      const int4 v = *reinterpret_cast<const int4*>(rows + f);
      pos += (v.x > re || (v.x == re && f < e)) + (v.y > re || (v.y == re && f + 1 < e)) +
             (v.z > re || (v.z == re && f + 2 < e)) + (v.w > re || (v.w == re && f + 3 < e));
    }
    o.order[pos] = (uint16_t)e;
  }
  __syncthreads();
  // this XCD's tiles per sorted position, then their exclusive prefix
  const int p0 = tid * PER;
  int cnt[PER];
  int local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int p = p0 + j;
    cnt[j] = p < E ? (rows[o.order[p]] + BM - 1) / BM * gmm_units_on(p, ntile, xcd) : 0;
    local += cnt[j];
  }
  scan_buf[tid] = local;
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
    const int add = tid >= off ? scan_buf[tid - off] : 0;
    __syncthreads();
    scan_buf[tid] += add;
    __syncthreads();
  }
  int run = scan_buf[tid] - local;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if (p0 + j < E) o.prefix[p0 + j] = run;
    run += cnt[j];
  }
  if (tid == NT - 1) o.prefix[E] = scan_buf[tid];
  __syncthreads();
}

static_assert((kMaxGmmExperts + 4 + GmmCfg::THREADS) * 4 <= GmmCfg::kBytes,
              "the order's work space fits the K ring");

struct GmmTile {
  int e, mcount, nt, mt, row_lo, row_hi, row0;
  int64_t n0;
};

// Tile s (0 <= s < o.prefix[E]) of this XCD's sequence.
__device__ __forceinline__ GmmTile gmm_tile_at(const GmmI8Args& a, const GmmOrder& o, int ntile,
                                               int xcd, int s) {
  GmmTile t;
  int lo = 0, hi = a.E;   // the largest p with prefix[p] <= s; it has tiles here
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (o.prefix[mid] <= s) lo = mid; else hi = mid;
  }
  t.e = o.order[lo];
  t.row_lo = gmm_row_of(a, t.e);
  const int rh = gmm_row_of(a, t.e + 1);
  t.row_hi = rh < t.row_lo ? t.row_lo : rh;
  t.mcount = (t.row_hi - t.row_lo + GmmCfg::BM - 1) / GmmCfg::BM;
  const int r = s - o.prefix[lo];
  t.nt = gmm_first_nt(lo, ntile, xcd) + kNumXcd * (r / t.mcount);
  t.mt = r % t.mcount;
  t.row0 = t.row_lo + t.mt * GmmCfg::BM;
  t.n0 = (int64_t)t.nt * GmmCfg::BN;
  return t;
}

// K stages [k0, k1) of tile t into acc (which it does not clear); kst =
// stages of the whole K.  Writes rowinfo (barrier inside); *ar: this
// thread's row scale (threads < BM), read while the loop runs.
__device__ __forceinline__ void gmm_tile_mainloop(const GmmI8Args& a, const GmmTile& t, int k0,
                                                  int k1, int kst, uint8_t* smem, int* rowinfo,
                                                  GmmAcc& acc, float* ar) {
  typedef GmmCfg C;
  constexpr int BN = C::BN, BM = C::BM;
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;
  if (tid < BM) rowinfo[tid] = (t.row0 + tid < t.row_hi) ? t.row0 + tid : -1;
  __syncthreads();
  const int64_t kshift = (int64_t)k0 * C::ROWB;        // bytes of K before stage k0
  const uint8_t* Wb = reinterpret_cast<const uint8_t*>(a.W) + (int64_t)t.e * a.N * a.K + kshift;
  // packed weights: this n-tile's blocks (tiles of kPackRows == BN rows), from stage k0
  const uint8_t* Wp = reinterpret_cast<const uint8_t*>(a.W) +
                      (((int64_t)t.e * packed_tiles(a.N, 0) + t.nt) * packed_kstages(a.K, 1) + k0) *
                          kPackBlockBytes;
  const uint8_t* rowp[C::NI];
  uint32_t pk_mask = 0;
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int q = wave * C::NI + j;
    const int r = q * 16 + (lane >> 2);
    if (r < BN && a.w_packed) {
      rowp[j] = Wp + q * 1024 + lane * 16;
      pk_mask |= 1u << j;
    } else if (r < BN) {
      const int64_t n = t.n0 + r;
      rowp[j] = Wb + (n < a.N ? n : 0) * a.K;
    } else {
      const int m = rowinfo[r - BN];
      rowp[j] = reinterpret_cast<const uint8_t*>(a.X) + (int64_t)(m < 0 ? t.row_lo : m) * a.K +
                kshift;
    }
  }
  // the only reader of this weight slice streams it with the non-temporal hint
  if (t.mcount == 1 && k0 == 0 && k1 == kst && pk_mask) pk_mask |= kPkStream;
  constexpr int WROWS = BN / C::WN;
  int wrow[C::RB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) wrow[rb] = wn * WROWS + rb * 32;
  const int tcol0 = wm * (BM / C::WM);
  const int live_m = t.row_hi - t.row0 < BM ? t.row_hi - t.row0 : BM;
  if (tid < BM && rowinfo[tid] >= 0) *ar = a.sx[rowinfo[tid]];
  // the last stage of K may be partial; earlier cut points are whole stages
  const int64_t kbytes = k1 == kst ? a.K - kshift : (int64_t)(k1 - k0) * C::ROWB;
  mainloop_dma_live<C, 1>(smem, rowp, pk_mask, kbytes, wrow, tcol0, live_m, acc);
}

// Epilogue through LDS: the fp16 tile in [token row][column] order in the
// drained K ring, then each row's BN columns as whole 16-byte pieces
// (straight from the MFMA layout each store would cover 32 rows x 8 bytes).
// When the whole tile does not fit the ring it goes in passes of one wave
// row (BM / WM token rows) each.
__device__ __forceinline__ void gmm_tile_epilogue(const GmmI8Args& a, const GmmTile& t,
                                                  const int* rowinfo, const GmmAcc& acc,
                                                  uint8_t* smem, float ar) {
  typedef GmmCfg C;
  constexpr int BN = C::BN, BM = C::BM, NT = C::THREADS;
  constexpr int PITCH = BN * 2 + 16, LPR = BN * 2 / 16, RPP = NT / LPR;
  constexpr bool kWhole = BM * PITCH + BM * 4 <= C::kBytes;
  constexpr int PR = kWhole ? BM : BM / C::WM;   // rows staged per pass
  static_assert(PR * PITCH + BM * 4 <= C::kBytes && NT % LPR == 0 && PR % RPP == 0 && BM <= NT,
                "staged GMM epilogue shape");
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::WN, wm = wave / C::WN;
  constexpr int WROWS = BN / C::WN;
  const int tcol0 = wm * (BM / C::WM);
  float* s_a = reinterpret_cast<float*>(smem + PR * PITCH);
  __syncthreads();                            // every wave has left the K ring
  if (tid < BM) s_a[tid] = ar;
  __syncthreads();
  const int rsub = 4 * (lane >> 5);
  const float* swe = a.sw + (int64_t)t.e * a.N;
  uint8_t* Yb = reinterpret_cast<uint8_t*>(a.Y);
  const int ch = tid % LPR;
  const int64_t col = t.n0 + ch * 8;          // 8 columns; N is a multiple of 16
#pragma unroll
  for (int p = 0; p < BM / PR; ++p) {
    if (kWhole || wm == p) {                  // this pass's rows: [p * PR, p * PR + PR)
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) {
        const int trow = tcol0 + cb * 32 + (lane & 31);
        const float sx = s_a[trow];
        uint8_t* dst = smem + (trow - p * PR) * PITCH;
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          const i32x16_t v = acc[rb][cb];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = wn * WROWS + rb * 32 + 8 * g + rsub;
            const int64_t n = t.n0 + c;
            const f32x4_t sw = *reinterpret_cast<const f32x4_t*>(swe + (n < a.N ? n : 0));   // past N: never stored
            *reinterpret_cast<uint2*>(dst + c * 2) = make_uint2(
                pack_f16x2((float)v[4 * g] * sx * sw[0], (float)v[4 * g + 1] * sx * sw[1]),
                pack_f16x2((float)v[4 * g + 2] * sx * sw[2], (float)v[4 * g + 3] * sx * sw[3]));
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int r0 = 0; r0 < PR; r0 += RPP) {
      const int r = r0 + tid / LPR;
      const int m = rowinfo[p * PR + r];
      if (m < 0 || col >= a.N) continue;
      *reinterpret_cast<u32x4_t*>(Yb + ((int64_t)m * a.N + col) * 2) =
          *reinterpret_cast<const u32x4_t*>(smem + r * PITCH + ch * 16);
    }
    if (p + 1 < BM / PR) __syncthreads();     // the next pass overwrites the staged rows
  }
}

__device__ __forceinline__ void gmm_acc_clear(GmmAcc& acc) {
#pragma unroll
  for (int rb = 0; rb < GmmCfg::RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < GmmCfg::CB; ++cb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0;
}

// One tile per workgroup (a grid of every possible tile; the surplus exits).
// OCC workgroups per CU: ask for OCC * waves / 4 waves per SIMD.
__global__ void __launch_bounds__(GmmCfg::THREADS, GmmCfg::OCC * GmmCfg::THREADS / 256)
gmm_i8_tile_kernel(GmmI8Args a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ GmmOrder order;
  __shared__ int rowinfo[GmmCfg::BM];
  const int ntile = (int)((a.N + GmmCfg::BN - 1) / GmmCfg::BN);
  const int xcd = (int)blockIdx.x % kNumXcd, slot = (int)blockIdx.x / kNumXcd;
  gmm_build_order(a, ntile, xcd, order, reinterpret_cast<int*>(smem));
  if (slot >= order.prefix[a.E]) return;
  const GmmTile t = gmm_tile_at(a, order, ntile, xcd, slot);
  const int kst = (int)((a.K + GmmCfg::ROWB - 1) / GmmCfg::ROWB);
  GmmAcc acc;
  gmm_acc_clear(acc);
  float ar = 0.0f;
  gmm_tile_mainloop(a, t, 0, kst, kst, smem, rowinfo, acc, &ar);
  gmm_tile_epilogue(a, t, rowinfo, acc, smem, ar);
}

// ---------------------------------------------------------------------------
// Expert-wide tiles (bf16).  The alignment pads each expert to 32-row blocks
// and one tile covers up to kWideMaxBlk consecutive blocks of one expert
// (every block of an expert with up to 320 pairs) against 256 weight rows,
// so a weight slice is streamed once for all of the expert's rows, and the
// tiles of one expert's n-tiles run side by side and share its token rows in
// L2.  One workgroup per CU (8 waves of 64 weight rows x up to 160 tokens).
// Weights and tokens have rings of their own: kWideNW weight stages (they
// come from HBM, so they are issued kWideNW - 1 stages ahead) and kWideNT
// token stages (token rows are mostly L2 hits).  Token pieces past the
// tile's blocks are not loaded at all (each wave's count of loads per stage
// is then smaller, and its waits count exactly what it issued).
#ifndef MOE_WIDE_NW
#define MOE_WIDE_NW 4
#endif
#ifndef MOE_WIDE_NT
#define MOE_WIDE_NT 4
#endif
constexpr int kWideBN = 256;
constexpr int kWideBlk = kWideBlockRows;
constexpr int kWideMaxBlk = kWideMaxBlocks;
constexpr int kWideBM = kWideBlk * kWideMaxBlk;            // token rows of a full tile
constexpr int kWideWN = 4, kWideWM = 2, kWideThreads = 64 * kWideWN * kWideWM;
constexpr int kWideNW = MOE_WIDE_NW, kWideNT = MOE_WIDE_NT;
static_assert(kWideNW >= kWideNT && kWideNT >= 2, "weight stages go out no later than token stages");
constexpr int kWideRowB = 64;                               // K bytes per row per stage
constexpr int kWideWStage = kWideBN * kWideRowB;            // 16 KiB
constexpr int kWideTStage = kWideBM * kWideRowB;            // 20 KiB
constexpr int kWideLds = kWideNW * kWideWStage + kWideNT * kWideTStage;
constexpr int kWideRB = kWideBN / kWideWN / 32;             // 2
constexpr int kWideCB = (kWideMaxBlk + kWideWM - 1) / kWideWM;   // token blocks per wave
constexpr int kWideWP = kWideBN / 16 / (kWideWN * kWideWM); // 2 weight pieces per wave
constexpr int kWideTP = (kWideBM / 16 + (kWideWN * kWideWM) - 1) / (kWideWN * kWideWM);   // <= 3
static_assert(kWideBN == kPackRows, "a wide tile's weight rows are one packed tile");
static_assert(kWideLds + 2 * kWideBM * 4 <= 160 * 1024, "rings, row info and row weights of the wide tile");

// Tile table of a layer: t[0] = number of tiles; tile j: t[1 + 3 j] = expert,
// t[2 + 3 j] = first block, t[3 + 3 j] = blocks (1..kWideMaxBlk).  An expert
// of nb blocks gets ceil(nb / kWideMaxBlk) tiles of nearly equal size.
constexpr int kWidePrepThreads = kWidePrepMaxExperts;

__global__ void __launch_bounds__(kWidePrepThreads)
wide_prep_kernel(const int32_t* __restrict__ expert_ids, const int32_t* __restrict__ total, int E,
                 int nblk_max, int32_t* __restrict__ table) {
  __shared__ int cnt[kWidePrepThreads], first[kWidePrepThreads], scan[kWidePrepThreads];
  const int tid = threadIdx.x;
  int nblk = *total / kWideBlk;
  nblk = nblk < nblk_max ? nblk : nblk_max;
  cnt[tid] = 0;
  first[tid] = 0;
  __syncthreads();
  for (int b = tid; b < nblk; b += kWidePrepThreads) {
    const int e = expert_ids[b];
    if (e < 0 || e >= E) continue;
    atomicAdd(&cnt[e], 1);
    if (b == 0 || expert_ids[b - 1] != e) first[e] = b;   // an expert's blocks are contiguous
  }
  __syncthreads();
  const int nt = tid < E ? (cnt[tid] + kWideMaxBlk - 1) / kWideMaxBlk : 0;
  scan[tid] = nt;
  __syncthreads();
  for (int off = 1; off < kWidePrepThreads; off <<= 1) {
    const int add = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  const int start = scan[tid] - nt;
  for (int i = 0; i < nt; ++i) {
    const int j = start + i;
    const int b0 = first[tid] + (int)((int64_t)i * cnt[tid] / nt);
    const int b1 = first[tid] + (int)((int64_t)(i + 1) * cnt[tid] / nt);
    table[1 + 3 * j] = tid;
    table[2 + 3 * j] = b0;
    table[3 + 3 * j] = b1 - b0;
  }
  if (tid == kWidePrepThreads - 1) table[0] = scan[tid];
}

// Loads of one stage by this wave: nt token pieces (1 KiB each; positions
// q = wave + 8 i) and kWideWP weight pieces (q = wave * kWideWP + i).
// Order in the instruction stream: tokens, then weights.
struct WideSrc {
  const uint8_t* w[kWideWP];   // this lane's 16 bytes of stage 0 of each weight piece
  const uint8_t* t[kWideTP];   // this lane's token row start of each token piece
  uint32_t wlds[kWideWP], tlds[kWideTP];   // LDS byte offset of each piece in its ring stage 0
  int nt;                      // token pieces of this wave (wave-uniform)
  bool packed, stream;         // packed weights; non-temporal weight loads
};

// wait until at most N of this wave's loads are outstanding, then barrier
// (n is wave-uniform; the most a wave can have issued after a stage's token
// loads is (kWideNT - 2) * (kWideTP + kWideWP))
static_assert((kWideNT - 2) * (kWideTP + kWideWP) <= 15, "wide_wait covers 0..15");
__device__ __forceinline__ void wide_wait(int n) {
  switch (n) {
    case 0: wait_vm_barrier<0>(); break;
    case 1: wait_vm_barrier<1>(); break;
    case 2: wait_vm_barrier<2>(); break;
    case 3: wait_vm_barrier<3>(); break;
    case 4: wait_vm_barrier<4>(); break;
    case 5: wait_vm_barrier<5>(); break;
    case 6: wait_vm_barrier<6>(); break;
    case 7: wait_vm_barrier<7>(); break;
    case 8: wait_vm_barrier<8>(); break;
    case 9: wait_vm_barrier<9>(); break;
    case 10: wait_vm_barrier<10>(); break;
    case 11: wait_vm_barrier<11>(); break;
    case 12: wait_vm_barrier<12>(); break;
    case 13: wait_vm_barrier<13>(); break;
    case 14: wait_vm_barrier<14>(); break;
    default: wait_vm_barrier<15>(); break;
  }
}

// K loop of a wide tile: stages [0, nk) of kbytes bytes of K.  ncb: this
// wave's token blocks (its accumulators beyond them stay untouched).
template <int KIND, int NCB>
__device__ __forceinline__ void wide_mainloop(uint8_t* smem, const WideSrc& src, int64_t kbytes,
                                              const int (&wrow)[kWideRB], int tcol0, bool w_issued,
                                              typename Mma<KIND>::acc_t (&acc)[kWideRB][kWideCB]) {
  const int tid = tile_tid(), lane = tid & 63;
  const uint32_t wbase = lds_addr(smem), tbase = wbase + kWideNW * kWideWStage;
  const int nk = (int)((kbytes + kWideRowB - 1) / kWideRowB);
  const int chunk_pos = lane & 3;
  const int nw = kWideWP, ntw = __builtin_amdgcn_readfirstlane(src.nt);

  // token piece i of stage kt (if this wave has it)
  auto issue_t1 = [&](int kt, int i) {
    if (i < ntw) {
      const uint32_t st = tbase + (uint32_t)((kt % kWideNT) * kWideTStage);
      const int64_t koff = (int64_t)kt * kWideRowB;
      const int row = (int)(src.tlds[i] / kWideRowB) + (lane >> 2);
      const int c = chunk_pos ^ ((row >> 2) & 3);
      const int64_t off = koff + c * 16 < kbytes ? koff + c * 16 : 0;   // past K: row start
      dma16(__builtin_amdgcn_readfirstlane(st + src.tlds[i]), src.t[i] + off);
    }
  };
  // weight piece i of stage kt
  auto issue_w1 = [&](int kt, int i) {
    const uint32_t st = wbase + (uint32_t)((kt % kWideNW) * kWideWStage);
    const int64_t koff = (int64_t)kt * kWideRowB;
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(st + src.wlds[i]);
    if (src.packed) {
      const uint8_t* g = src.w[i] + (int64_t)kt * kPackBlockBytes;
      if (src.stream) dma16_nt(m0, g); else dma16(m0, g);
    } else {
      const int row = (int)(src.wlds[i] / kWideRowB) + (lane >> 2);
      const int c = chunk_pos ^ ((row >> 2) & 3);
      dma16(m0, src.w[i] + (koff + c * 16 < kbytes ? koff + c * 16 : 0));
    }
  };
  auto issue_t = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kWideTP; ++i) issue_t1(kt, i);
  };
  auto issue_w = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kWideWP; ++i) issue_w1(kt, i);
  };
  // zero the chunks of a partial stage that lie past K (after its loads landed)
  auto zero_tail = [&](int kt) {
    const int64_t koff = (int64_t)kt * kWideRowB;
    uint8_t* ws = smem + (kt % kWideNW) * kWideWStage;
    uint8_t* ts = smem + kWideNW * kWideWStage + (kt % kWideNT) * kWideTStage;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    if (!src.packed) {
#pragma unroll
      for (int i = 0; i < kWideWP; ++i) {
        const int row = (int)(src.wlds[i] / kWideRowB) + (lane >> 2);
        if (koff + (chunk_pos ^ ((row >> 2) & 3)) * 16 >= kbytes)
          *reinterpret_cast<u32x4_t*>(ws + src.wlds[i] + lane * 16) = z;
      }
    }
#pragma unroll
    for (int i = 0; i < kWideTP; ++i) {
      if (i < ntw) {
        const int row = (int)(src.tlds[i] / kWideRowB) + (lane >> 2);
        if (koff + (chunk_pos ^ ((row >> 2) & 3)) * 16 >= kbytes)
          *reinterpret_cast<u32x4_t*>(ts + src.tlds[i] + lane * 16) = z;
      }
    }
  };
  // Issue schedule: the prologue issues W(0 .. NW - 2) (unless the previous
  // tile of this workgroup already did, before its epilogue), then
  // T(0 .. NT - 2); iteration i (its stage published, every wave done with
  // stage i - 1) issues W(i + NW - 1), then T(i + NT - 1), into the buffers
  // of stage i - 1.  Loads complete in issue order, so stage s is in when
  // the loads issued after T(s) are all that may be outstanding: the later
  // prologue T's and the W and T of the iterations from max(0, s - NT + 2)
  // to s - 1 (W(s) went out before T(s), as NW >= NT).  Stores issued in
  // between (the previous tile's epilogue) also count in vmcnt; they only
  // make a wait longer.
  auto n_after = [&](int s) {
    int n = 0;
#pragma unroll
    for (int i = s - kWideNT + 2; i < s; ++i)
      if (i >= 0) n += (i + kWideNT - 1 < nk ? ntw : 0) + (i + kWideNW - 1 < nk ? nw : 0);
#pragma unroll
    for (int j = 1; j <= kWideNT - 2; ++j)
      if (j > s && j < nk) n += ntw;
    return n;
  };
  const bool partial = (kbytes % kWideRowB) != 0;
  auto publish = [&](int s) {
    if (partial && s == nk - 1) {
      wide_wait(0);
      zero_tail(s);
      __syncthreads();
    } else {
      wide_wait(n_after(s));
    }
  };
  if (!w_issued) {
    for (int i = 0; i < kWideNW - 1 && i < nk; ++i) issue_w(i);
  }
  for (int i = 0; i < kWideNT - 1 && i < nk; ++i) issue_t(i);

  const int swz = ((lane & 31) >> 2) & 3;
  auto load_frags = [&](int kt, int ks, u32x4_t (&af)[kWideRB], u32x4_t (&bf)[kWideCB]) {
    const uint8_t* ws = smem + (kt % kWideNW) * kWideWStage + (lane & 31) * kWideRowB;
    const uint8_t* ts = smem + kWideNW * kWideWStage + (kt % kWideNT) * kWideTStage +
                        (lane & 31) * kWideRowB;
    const int pos = ((ks * 2 + (lane >> 5)) ^ swz) * 16;
    if constexpr (NCB > 0) {
#pragma unroll
      for (int rb = 0; rb < kWideRB; ++rb)
        af[rb] = *reinterpret_cast<const u32x4_t*>(ws + wrow[rb] * kWideRowB + pos);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      bf[cb] = *reinterpret_cast<const u32x4_t*>(ts + (tcol0 + cb * 32) * kWideRowB + pos);
  };
  // The MFMAs of one K step, token block by token block; after block cb the
  // load pieces that the schedule puts there (pw: weight piece, pt: token
  // piece, -1 none).  The scheduling barriers keep the order.
  auto step = [&](const u32x4_t (&af)[kWideRB], const u32x4_t (&bf)[kWideCB], int kw, int ktk,
                  auto sched) {
#pragma unroll
    for (int cb = 0; cb < (NCB > 0 ? NCB : 1); ++cb) {
      if (cb < NCB) {
#pragma unroll
        for (int rb = 0; rb < kWideRB; ++rb) acc[rb][cb] = Mma<KIND>::run(af[rb], bf[cb], acc[rb][cb]);
      }
      __builtin_amdgcn_sched_barrier(0);
      sched(cb, kw, ktk);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // K step 0 of a stage carries the weight pieces, step 1 the token pieces,
  // one after each of the first token blocks (all after the last block when
  // the wave has fewer blocks than pieces)
  constexpr int kLast = (NCB > 0 ? NCB : 1) - 1;
  auto sched_w = [&](int cb, int kw, int) {
#pragma unroll
    for (int i = 0; i < kWideWP; ++i)
      if (kw >= 0 && (i < kLast ? cb == i : cb == kLast)) issue_w1(kw, i);
  };
  auto sched_t = [&](int cb, int, int ktk) {
#pragma unroll
    for (int i = 0; i < kWideTP; ++i)
      if (ktk >= 0 && (i < kLast ? cb == i : cb == kLast)) issue_t1(ktk, i);
  };
  // one set of fragments (the accumulators take most of the registers; the
  // other wave on the SIMD covers the LDS latency)
  u32x4_t af[kWideRB], bf[kWideCB];
  publish(0);
  load_frags(0, 0, af, bf);
  // Iteration kt refills the buffers of stage kt - 1 (every wave left them
  // at the barrier before it) with W(kt + NW - 1), then T(kt + NT - 1).  The
  // loads go out one by one between the MFMAs: when the memory queues are
  // full a load waits at issue, and the MFMAs already issued keep the matrix
  // core busy meanwhile (issued in one burst after the barrier, the loads
  // held every wave of the CU at once).
  for (int kt = 0; kt < nk; ++kt) {
    step(af, bf, kt + kWideNW - 1 < nk ? kt + kWideNW - 1 : -1, -1, sched_w);
    load_frags(kt, 1, af, bf);
    step(af, bf, -1, kt + kWideNT - 1 < nk ? kt + kWideNT - 1 : -1, sched_t);
    if (kt + 1 < nk) {
      publish(kt + 1);
      load_frags(kt + 1, 0, af, bf);
    }
  }
}

// Runs the K loop specialised for this wave's number of token blocks.
template <int KIND>
__device__ __forceinline__ void wide_mainloop_live(uint8_t* smem, const WideSrc& src,
                                                   int64_t kbytes, const int (&wrow)[kWideRB],
                                                   int tcol0, int ncb, bool w_issued,
                                                   typename Mma<KIND>::acc_t (&acc)[kWideRB][kWideCB]) {
  static_assert(kWideCB <= 5, "wide_mainloop_live dispatches up to 5 token blocks");
  switch (__builtin_amdgcn_readfirstlane(ncb)) {
    case 5: return wide_mainloop<KIND, 5>(smem, src, kbytes, wrow, tcol0, w_issued, acc);
    case 4: return wide_mainloop<KIND, 4>(smem, src, kbytes, wrow, tcol0, w_issued, acc);
    case 3: return wide_mainloop<KIND, 3>(smem, src, kbytes, wrow, tcol0, w_issued, acc);
    case 2: return wide_mainloop<KIND, 2>(smem, src, kbytes, wrow, tcol0, w_issued, acc);
    case 1: return wide_mainloop<KIND, 1>(smem, src, kbytes, wrow, tcol0, w_issued, acc);
    default: return wide_mainloop<KIND, 0>(smem, src, kbytes, wrow, tcol0, w_issued, acc);
  }
}

// A wide tile: expert e, its blocks [b0, b0 + nb), n-tile nt, and whether it
// is the only tile of its weight slice; valid = inside the alignment's
// blocks and experts (a bad table entry is skipped, not read).
struct WideTile {
  int e, b0, nb, nt;
  bool stream, valid;
};

__device__ __forceinline__ WideTile wide_tile_at(const MoeGemmArgs& a, const int32_t* table,
                                                 int ntiles, int ntile, int L) {
  WideTile w;
  const int j = L / ntile;
  w.nt = L % ntile;
  w.e = table[1 + 3 * j];
  w.b0 = table[2 + 3 * j];
  w.nb = table[3 + 3 * j];
  w.valid = !(w.e < 0 || w.e >= a.E || w.b0 < 0 || w.nb < 1 || w.nb > kWideMaxBlk ||
              (int64_t)(w.b0 + w.nb) * kWideBlk > a.max_padded);
  w.stream = a.b_packed != 0 && (j == 0 || table[1 + 3 * (j - 1)] != w.e) &&
             (j + 1 >= ntiles || table[1 + 3 * (j + 1)] != w.e);
  return w;
}

// This wave's weight pieces of tile w (stage-0 addresses); rows past the
// matrix read row 0.
template <int EPI, int KIND>
__device__ __forceinline__ void wide_weight_src(const MoeGemmArgs& a, const WideTile& w, int wave,
                                                int lane, WideSrc& src) {
  constexpr int kElem = KIND ? 1 : 2;
  src.packed = a.b_packed != 0;
  src.stream = w.stream;
  const int64_t wrow_bytes = a.K * kElem;
  const int64_t c0 = (int64_t)w.nt * (EPI ? kWideBN / 2 : kWideBN);
  const uint8_t* Bw = reinterpret_cast<const uint8_t*>(a.B) + (int64_t)w.e * a.N * wrow_bytes;
  const uint8_t* Bp = reinterpret_cast<const uint8_t*>(a.B) +
                      ((int64_t)w.e * packed_tiles(a.N, EPI) + w.nt) * packed_kstages(a.K, kElem) *
                          kPackBlockBytes;
#pragma unroll
  for (int i = 0; i < kWideWP; ++i) {
    const int q = wave * kWideWP + i;
    src.wlds[i] = (uint32_t)(q * 1024);
    if (src.packed) {
      src.w[i] = Bp + q * 1024 + lane * 16;
    } else {
      const int64_t g = moe_weight_row<kWideBN, EPI>(a, c0, q * 16 + (lane >> 2));
      src.w[i] = Bw + (g < 0 ? 0 : g) * wrow_bytes;
    }
  }
}

// The weight loads of stages 0 .. NW - 2 of a tile (the K loop's prologue
// otherwise issues them), this wave's pieces, in the loop's order.
__device__ __forceinline__ void wide_prefetch_w(uint8_t* smem, const WideSrc& src, int64_t kbytes) {
  const int lane = tile_tid() & 63, chunk_pos = lane & 3;
  const uint32_t wbase = lds_addr(smem);
  const int nk = (int)((kbytes + kWideRowB - 1) / kWideRowB);
  for (int kt = 0; kt < kWideNW - 1 && kt < nk; ++kt) {
#pragma unroll
    for (int i = 0; i < kWideWP; ++i) {
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(
          wbase + (uint32_t)(kt * kWideWStage) + src.wlds[i]);
      if (src.packed) {
        const uint8_t* g = src.w[i] + (int64_t)kt * kPackBlockBytes;
        if (src.stream) dma16_nt(m0, g); else dma16(m0, g);
      } else {
        const int64_t koff = (int64_t)kt * kWideRowB;
        const int row = (int)(src.wlds[i] / kWideRowB) + (lane >> 2);
        const int c = chunk_pos ^ ((row >> 2) & 3);
        dma16(m0, src.w[i] + (koff + c * 16 < kbytes ? koff + c * 16 : 0));
      }
    }
  }
}

// EPI 1: gate_up with the SiLU*up epilogue, bf16 h in sorted order;
// EPI 0: down times the routing weight, bf16 rows in pair order.
// KIND 0: bf16 tokens and weights; KIND 1: int8 tokens and weights, exact
// int32 sums times the row scale (a_scales) and the channel scale (b_scales).
// One workgroup per CU, persistent: the grid is 8 x S workgroups, and
// workgroup (XCD x = id % 8, slot id / 8) takes positions slot, slot + S, ...
// of XCD x's contiguous run of tiles, so the n-tiles of one expert tile run
// side by side on one XCD and share the expert's token rows in L2.  Once a
// tile's K loop is done its workgroup issues the next tile's first weight
// stages, then runs the epilogue (staged in the LDS the next tile does not
// use yet), so the weight stream goes on through epilogues and tile changes.
template <int EPI, int KIND>
__global__ void __launch_bounds__(kWideThreads, 2)
moe_gemm_wide_kernel(MoeGemmArgs a, const int32_t* __restrict__ table) {
  typedef typename Mma<KIND>::acc_t Acc;
  constexpr int kElem = KIND ? 1 : 2;                  // bytes per operand element
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int rowinfo[kWideBM];
  __shared__ float s_w[kWideBM];
  __shared__ float s_as[KIND ? kWideBM : 1];           // int8: row scales of the tile
  __shared__ __attribute__((aligned(16))) float s_bs[KIND ? kWideBN : 4];   // and channel scales
  // epilogue staging: the last weight stage and the token ring (the next
  // tile's weight stages 0 .. NW - 2 are in flight meanwhile)
  uint8_t* stage_lds = smem + (kWideNW - 1) * kWideWStage;
  constexpr int kStageBytes = kWideWStage + kWideNT * kWideTStage;
  const int ntile = moe_ntiles<kWideBN, EPI>(a);
  // tiles in the table, never more than its room: one per block at most
  const int64_t nblk = a.max_padded / kWideBlk;
  const int ntiles = (int)(table[0] < 0 ? 0 : (table[0] < nblk ? table[0] : nblk));
  const int live = ntiles * ntile;
  const int xcd = (int)blockIdx.x % kNumXcd;
  const int q = live / kNumXcd, r = live % kNumXcd;
  const int run0 = xcd * q + (xcd < r ? xcd : r), runlen = q + (xcd < r ? 1 : 0);
  const int tid = tile_tid(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % kWideWN, wm = wave / kWideWN;
  const int64_t wrow_bytes = a.K * kElem;
  int wrow[kWideRB];
  wave_rows<kWideBN, kWideWN, kWideRB, EPI>(wn, wrow);
  static_assert(kWideBM <= kWideThreads, "one row of row info per thread");
  // pair index of tile row tid of tile w (-1: padding or out of range)
  auto row_pair = [&](const WideTile& w) {
    int p = -1;
    if (tid < w.nb * kWideBlk) {
      p = a.sorted_ids[(int64_t)w.b0 * kWideBlk + tid];
      if (p < 0 || p >= a.num_valid) p = -1;
    }
    return p;
  };
  const int S = (int)gridDim.x / kNumXcd, slot = (int)blockIdx.x / kNumXcd;
  int pos = slot;
  while (pos < runlen && !wide_tile_at(a, table, ntiles, ntile, run0 + pos).valid) pos += S;
  if (pos >= runlen) return;
  WideTile w = wide_tile_at(a, table, ntiles, ntile, run0 + pos);
  int pair = row_pair(w);                              // this thread's row of the tile
  bool w_issued = false;
  for (;;) {
    const int e = w.e, nb = w.nb, nt = w.nt;
    const int nrows = nb * kWideBlk;
    const int64_t s0 = (int64_t)w.b0 * kWideBlk;      // first sorted position
    if (tid < kWideBM) rowinfo[tid] = pair;
    __syncthreads();
    MoeTile t;
    t.e = e; t.blk = w.b0; t.nt = nt; t.s0 = s0;
    t.c0 = (int64_t)nt * (EPI ? kWideBN / 2 : kWideBN);
    t.solo = 0;
    // int8: the tile's row and channel scales into LDS now, so that the
    // epilogue does not wait on global loads queued behind the next tile's
    // weight loads (loads complete in issue order)
    if constexpr (KIND != 0) {
      if (tid < kWideBM) {
        const int p = rowinfo[tid];
        s_as[tid] = p < 0 ? 0.0f
                          : a.a_scales[a.a_rows == 0 ? (int64_t)(p / a.a_row_div) : s0 + tid];
      }
      if (tid < kWideBN) {
        // weight row tid of the tile: gate / up channel (SiLU) or channel c0 + tid
        const int64_t n = EPI ? (tid < kWideBN / 2 ? t.c0 + tid : a.N / 2 + t.c0 + tid - kWideBN / 2)
                              : t.c0 + tid;
        s_bs[tid] = n < a.N ? a.b_scales[(int64_t)e * a.N + n] : 0.0f;
      }
      asm volatile("" ::: "memory");                  // the stores go out here, not later
    }
    WideSrc src;
    wide_weight_src<EPI, KIND>(a, w, wave, lane, src);
    const uint8_t* Ab = reinterpret_cast<const uint8_t*>(a.A);
    const int64_t arow_bytes = a.lda * kElem;
    src.nt = 0;
#pragma unroll
    for (int i = 0; i < kWideTP; ++i) {
      const int qq = wave + i * (kWideWN * kWideWM);
      src.tlds[i] = (uint32_t)(qq * 1024);
      const int rrow = qq * 16 + (lane >> 2);
      if (qq * 16 < nrows) {
        src.nt = i + 1;
        const int p = rowinfo[rrow];
        const int p0 = rowinfo[0] < 0 ? 0 : rowinfo[0];  // row 0 of a tile is a pair
        const int64_t row = a.a_rows == 0 ? (int64_t)((p < 0 ? p0 : p) / a.a_row_div)
                                          : (p < 0 ? s0 : s0 + rrow);
        src.t[i] = Ab + row * arow_bytes;
      } else {
        src.t[i] = Ab;
      }
    }
    const int h = (nb + 1) / 2;                        // token blocks of wave row 0
    const int tcol0 = wm ? h * kWideBlk : 0;
    const int ncb = wm ? nb - h : h;
    // this thread's row weight (down), read while the K loop runs
    float wr = 1.0f;
    if (!EPI && a.topk_weights && tid < nrows && rowinfo[tid] >= 0)
      wr = a.topk_weights[rowinfo[tid]];
    Acc acc[kWideRB][kWideCB];
#pragma unroll
    for (int rb = 0; rb < kWideRB; ++rb)
#pragma unroll
      for (int cb = 0; cb < kWideCB; ++cb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[rb][cb][v] = 0;
    wide_mainloop_live<KIND>(smem, src, wrow_bytes, wrow, tcol0, ncb, w_issued, acc);

    // every wave has left the rings: the next tile's first weight stages go
    // out now and stream in while this tile's epilogue runs (its row info is
    // read now too)
    __syncthreads();
    int next = pos + S;
    while (next < runlen && !wide_tile_at(a, table, ntiles, ntile, run0 + next).valid) next += S;
    w_issued = next < runlen;
    WideTile wn_tile = w;
    if (w_issued) {
      wn_tile = wide_tile_at(a, table, ntiles, ntile, run0 + next);
      WideSrc nsrc;
      wide_weight_src<EPI, KIND>(a, wn_tile, wave, lane, nsrc);
      wide_prefetch_w(smem, nsrc, wrow_bytes);
      pair = row_pair(wn_tile);
    }

    // Epilogue through the token ring's LDS, whole 16-byte pieces of rows,
    // in passes of whole token blocks.  Scales (int8): the row's a_scales
    // entry and the channel's b_scales entry (1 for bf16, which leaves the
    // sums' bits as they are).  The thread index goes through an empty asm
    // statement so that nothing computed from it here is hoisted out of the
    // tile loop, where it would hold registers through the K loop.
    int etid = tid;
    asm volatile("" : "+v"(etid));
    const int elane = etid & 63;
    const int rsub = 4 * (elane >> 5);
    uint8_t* Cb = reinterpret_cast<uint8_t*>(a.C);
    const f32x4_t one4 = {1.0f, 1.0f, 1.0f, 1.0f};
    // The scale reads are volatile, so that they are not hoisted out of the
    // token-block loop (where the 8 column scale vectors would hold 32
    // registers beside the accumulators), through pointers typed as LDS: a
    // volatile read through a generic pointer compiles to a flat load, which
    // counts in vmcnt and so waits for the next tile's weight stages.
    typedef __attribute__((address_space(3))) const volatile float lds_cvf;
    typedef __attribute__((address_space(3))) const volatile f32x4_t lds_cvf4;
    auto row_scale = [&](int trow) -> float {   // trow a row of the tile
      if constexpr (KIND == 0) return 1.0f;
      return *(lds_cvf*)(s_as + trow);
    };
    auto col_scale = [&](int c) -> f32x4_t {    // weight rows c .. c + 3 of the tile
      if constexpr (KIND == 0) return one4;
      return *(lds_cvf4*)(s_bs + c);
    };
    if (!EPI && etid < kWideBM) s_w[etid] = wr;
    // pass p stages the token blocks [p * BPP, (p + 1) * BPP) of the tile
    constexpr int OUTC = EPI ? kWideBN / 2 : kWideBN;  // output columns of the tile
    constexpr int PITCH = OUTC * 2 + 16, LPR = OUTC * 2 / 16;
    constexpr int RPP = kWideThreads / LPR;
    constexpr int BPP = kStageBytes / (32 * PITCH) < kWideMaxBlk ? kStageBytes / (32 * PITCH)
                                                                 : kWideMaxBlk;
    static_assert(BPP >= 1, "one token block of the staged tile fits the staging space");
    const int npass = (nb + BPP - 1) / BPP;
    const int64_t Nout = EPI ? a.N / 2 : a.N;
    const int ch = etid % LPR;
    const int64_t col = t.c0 + ch * 8;
    const int blk0 = tcol0 / kWideBlk;                 // this wave's first token block
    for (int pass = 0; pass < npass; ++pass) {
      const int rbase = pass * BPP * kWideBlk;
      const int rend = nrows < rbase + BPP * kWideBlk ? nrows : rbase + BPP * kWideBlk;
      __syncthreads();
#pragma unroll
      for (int cb = 0; cb < kWideCB; ++cb) {
        const int bi = blk0 + cb - pass * BPP;
        if (cb < ncb && bi >= 0 && bi < BPP) {
          const int trow = tcol0 + cb * 32 + (elane & 31);
          const float as = row_scale(trow);
          uint8_t* dst = stage_lds + (trow - rbase) * PITCH;
          if constexpr (EPI) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = wrow[0] + 8 * g + rsub;   // output column t.c0 + c
              const f32x4_t gt = acc4(acc[0][cb], g, as, col_scale(wrow[0] + 8 * g + rsub));
              const f32x4_t up = acc4(acc[1][cb], g, as, col_scale(wrow[1] + 8 * g + rsub));
              *reinterpret_cast<uint2*>(dst + c * 2) = make_uint2(
                  pack_bf16x2(silu_f32(gt[0]) * up[0], silu_f32(gt[1]) * up[1]),
                  pack_bf16x2(silu_f32(gt[2]) * up[2], silu_f32(gt[3]) * up[3]));
            }
          } else {
            const float wt = s_w[trow];
            const float rf = KIND ? as * wt : wt;
#pragma unroll
            for (int rb = 0; rb < kWideRB; ++rb) {
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int c = wrow[rb] + 8 * g + rsub;
                const f32x4_t v = row4(acc[rb][cb], g, rf, col_scale(c));
                *reinterpret_cast<uint2*>(dst + c * 2) = make_uint2(
                    pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
              }
            }
          }
        }
      }
      __syncthreads();
      for (int r0 = rbase; r0 < rend; r0 += RPP) {
        const int rr = r0 + etid / LPR;
        if (rr >= rend || rowinfo[rr] < 0 || col >= Nout) continue;
        const int64_t crow = a.c_rows == 0 ? (int64_t)rowinfo[rr] : s0 + rr;
        *reinterpret_cast<u32x4_t*>(Cb + (crow * a.ldc + col) * 2) =
            *reinterpret_cast<const u32x4_t*>(stage_lds + (rr - rbase) * PITCH + ch * 16);
      }
    }
    __syncthreads();                                   // staging and rowinfo free again
    if (!w_issued) break;
    pos = next;
    w = wn_tile;
  }
}

// Dynamic LDS beyond 64 KiB has to be requested per kernel.
template <typename K>
hipError_t ensure_lds(K kernel, size_t bytes) {
  return raise_lds_limit(reinterpret_cast<const void*>(kernel), bytes);
}

template <class C, int EPI, bool TF32, int CDT, int KIND = 0>
hipError_t launch_tile_t(const MoeGemmArgs& a, hipStream_t stream) {
  const int64_t Nout = EPI ? a.N / 2 : a.N;
  const int64_t ncols = EPI ? C::BN / 2 : C::BN;
  const int64_t ntile = (Nout + ncols - 1) / ncols;
  const int64_t grid = (a.max_padded / C::BM) * ntile;
  if (grid == 0) return hipSuccess;
  void (*k)(MoeGemmArgs);
  if constexpr (TF32) k = moe_gemm_tile_kernel<C, EPI, CDT>;
  else k = moe_gemm_dma_kernel<C, EPI, CDT, KIND>;
  constexpr size_t lds = C::kBytes;
  const hipError_t st = ensure_lds(k, lds);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(C::THREADS), lds, stream, a);
  return hipGetLastError();
}

template <class C, int EPI, bool TF32>
hipError_t launch_tile_c(const MoeGemmArgs& a, hipStream_t s) {
  switch (a.c_dtype) {
    case 0: return launch_tile_t<C, EPI, TF32, 0>(a, s);
    case 1: return launch_tile_t<C, EPI, TF32, 1>(a, s);
    default: return launch_tile_t<C, EPI, TF32, 2>(a, s);
  }
}

// Tile configurations per block size.  bf16 tokens: direct-to-LDS loop,
// BN x BM with NSTAGE LDS stages; float32 tokens: register-staged loop.
template <int BM> struct TileFor;
// 256 x 128 tiles: 8 waves of 64 x 64, a 3-stage ring (72 KiB) and two
// workgroups per CU, so one workgroup's MFMAs run while the other waits at
// its barrier or for its loads (measured faster than one 256 x 256 tile per
// CU with 8 or 16 waves).
#ifndef MOE_T128_NSTAGE
#define MOE_T128_NSTAGE 3
#define MOE_T128_OCC 2
#endif
#ifndef MOE_T128_WN
#define MOE_T128_WN 4
#define MOE_T128_WM 2
#endif
#ifndef MOE_T128_BN
#define MOE_T128_BN 256
#endif
// 256 x 64 tiles (decode and small experts): 4 waves, a 3-stage ring (60 KiB)
// and two workgroups per CU: more weight bytes in flight per CU than one
// workgroup with a 4-stage ring (measured 1-4% faster on the decode layers).
#ifndef MOE_T64_NSTAGE
#define MOE_T64_NSTAGE 3
#define MOE_T64_OCC 2
#define MOE_T64_WN 2
#define MOE_T64_WM 2
#endif
template <> struct TileFor<64> {
  typedef DmaCfg<256, 64, MOE_T64_NSTAGE, MOE_T64_WN, MOE_T64_WM, MOE_T64_OCC, true> Dma;
  typedef Cfg<256, 64, 2, 2, MOE_TILE_NBUF> Regs;
};
template <> struct TileFor<128> {
  typedef DmaCfg<MOE_T128_BN, 128, MOE_T128_NSTAGE, MOE_T128_WN, MOE_T128_WM, MOE_T128_OCC> Dma;
  typedef Cfg<256, 128, 2, 2, MOE_TILE_NBUF> Regs;
};
template <> struct TileFor<256> {
  typedef DmaCfg<256, 256, MOE_T256_NSTAGE, MOE_T256_WN, MOE_T256_WM> Dma;   // 2 waves per SIMD
};

template <int BM>
hipError_t launch_tile_bm(const MoeGemmArgs& a, hipStream_t s) {
  typedef typename TileFor<BM>::Dma D;
  static_assert(D::BN % kPackRows == 0, "a tile is a whole number of packed tiles");
  if (a.b_packed && a.a_dtype == 0) return hipErrorInvalidValue;   // rejected by the ABI layer
  if (a.a_dtype == 3) {   // int8 tokens and weights; f32 or bf16 output
    if (a.c_dtype == 0)
      return a.epilogue ? launch_tile_t<D, 1, false, 0, 1>(a, s) : launch_tile_t<D, 0, false, 0, 1>(a, s);
    if (a.c_dtype == 1)
      return a.epilogue ? launch_tile_t<D, 1, false, 1, 1>(a, s) : launch_tile_t<D, 0, false, 1, 1>(a, s);
    return hipErrorInvalidValue;
  }
  if (a.a_dtype != 0)
    return a.epilogue ? launch_tile_c<D, 1, false>(a, s) : launch_tile_c<D, 0, false>(a, s);
  if constexpr (BM > 128) {
    return hipErrorInvalidValue;   // rejected by the ABI layer beforehand
  } else {
    typedef typename TileFor<BM>::Regs R;
    return a.epilogue ? launch_tile_c<R, 1, true>(a, s) : launch_tile_c<R, 0, true>(a, s);
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

int64_t wide_table_ints(int64_t max_padded) { return 1 + 3 * (max_padded / kWideBlk); }

hipError_t launch_wide_prep(const int32_t* expert_ids, const int32_t* total, int E,
                            int64_t max_padded, int32_t* table, hipStream_t stream) {
  if (E < 1 || E > kWidePrepThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wide_prep_kernel, dim3(1), dim3(kWidePrepThreads), 0, stream, expert_ids,
                     total, E, (int)(max_padded / kWideBlk), table);
  return hipGetLastError();
}

hipError_t raise_lds_limit(const void* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t st = hipGetDevice(&dev);
  if (st != hipSuccess) return st;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> raised;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = raised[std::make_pair(kernel, dev)];
  if (have >= bytes) return hipSuccess;
  st = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (st == hipSuccess) have = bytes;
  return st;
}

namespace {

constexpr int kMaxDevices = 64;

// Compute units of the current device, read once per device.
hipError_t current_device_cus(int* cus) {
  static std::atomic<int> cache[kMaxDevices] = {};
  int dev = 0;
  hipError_t st = hipGetDevice(&dev);
  if (st != hipSuccess) return st;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    st = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (st != hipSuccess) return st;
    if (v <= 0) return hipErrorInvalidDevice;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  *cus = v;
  return hipSuccess;
}

}  // namespace

hipError_t launch_moe_gemm_wide(const MoeGemmArgs& a, const int32_t* table, hipStream_t stream) {
  const bool i8 = a.a_dtype == 3;
  if (a.block_m != kWideBlk || (a.a_dtype != 1 && !i8) || a.c_dtype != 1 ||
      (a.epilogue && a.topk_weights) || (i8 && (!a.a_scales || !a.b_scales)))
    return hipErrorInvalidValue;   // the ABI layer checks these first
  // tiles: at most one per expert plus one per kWideMaxBlk blocks
  const int64_t nblk = a.max_padded / kWideBlk;
  const int64_t tiles = nblk / kWideMaxBlk + (a.E < nblk ? a.E : nblk);
  const int64_t ntile = a.epilogue ? (a.N / 2 + kWideBN / 2 - 1) / (kWideBN / 2)
                                   : (a.N + kWideBN - 1) / kWideBN;
  const int64_t max_tiles = tiles * ntile;
  if (max_tiles == 0) return hipSuccess;
  // one persistent workgroup per CU, the same number on each XCD
  int cus = 0;
  hipError_t st = current_device_cus(&cus);
  if (st != hipSuccess) return st;
  int64_t per_xcd = (cus + kNumXcd - 1) / kNumXcd;
  const int64_t need = (max_tiles + kNumXcd - 1) / kNumXcd;
  per_xcd = per_xcd < need ? per_xcd : need;
  const int64_t grid = per_xcd * kNumXcd;
  void (*k)(MoeGemmArgs, const int32_t*) =
      i8 ? (a.epilogue ? moe_gemm_wide_kernel<1, 1> : moe_gemm_wide_kernel<0, 1>)
         : (a.epilogue ? moe_gemm_wide_kernel<1, 0> : moe_gemm_wide_kernel<0, 0>);
  st = ensure_lds(k, kWideLds);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(k, dim3((unsigned)grid), dim3(kWideThreads), kWideLds, stream, a, table);
  return hipGetLastError();
}

hipError_t launch_gmm_int8(const GmmI8Args& a, hipStream_t stream) {
  typedef GmmCfg C;
  const int ntile = (int)((a.N + C::BN - 1) / C::BN);
  // Upper bound of m-tiles: every non-empty expert adds at most one partial
  // tile; an XCD gets at most ceil(ntile / 8) n-tiles of each expert.
  const int64_t mt_max = (a.M + C::BM - 1) / C::BM + a.E;
  const int64_t grid = mt_max * ((ntile + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid == 0 || a.M == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  constexpr size_t lds = C::kBytes;
  const hipError_t st = ensure_lds(gmm_i8_tile_kernel, lds);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(gmm_i8_tile_kernel, dim3((unsigned)grid), dim3(C::THREADS), lds, stream, a);
  return hipGetLastError();
}

}  // namespace moe

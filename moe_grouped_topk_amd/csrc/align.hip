// Alignment kernel: stable sort of (token, expert) pairs by expert with every
// expert's segment padded to a multiple of block_m.
//
// Semantics: mini-sglang "MoE and fused MoE", moe_align_block_size (stable
// argsort by expert, placeholder = number of pairs, one expert id per block).
//
// Two kernels, both keeping every total on the device.  The expert-parallel
// one (below) serves the usual sizes; this single 1024-thread workgroup (16
// waves) serves very large pair counts.  Wave w owns a contiguous chunk of
// the pairs.
//   pass 1: per-wave histograms counts[w][e] in LDS (LDS atomics), the ids
//           read in batches so many loads are in flight at once;
//   scan:   per expert, exclusive prefix over waves (so wave w knows where its
//           pairs of expert e start inside the segment), padded sizes, and an
//           exclusive scan over experts for the segment starts;
//   pass 2: each wave re-reads its chunk 64 pairs at a time; lanes holding
//           the same expert find each other with one ballot per bit of the
//           expert id, take their rank among themselves, and write their pair
//           index; the highest such lane advances the wave's cursor.  Chunks
//           are in pair order and ranks follow lane order, so the order
//           inside each segment is ascending pair index (stable).
//   tail:   placeholders, expert ids per block, the total, and the unused
//           tail of the buffers (placeholder / -1).

#include "common.hpp"
#include "launch.hpp"

namespace moe {

constexpr int kAlignThreads = 1024;
constexpr int kAlignWaves = kAlignThreads / kWave;
constexpr int kBatch = 16;   // ids per lane read together

__global__ void __launch_bounds__(kAlignThreads)
align_kernel(const int32_t* __restrict__ topk_ids, int P, int E, int B,
             int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
             int32_t* __restrict__ total_out, int max_padded) {
  extern __shared__ int smem[];
  int* counts = smem;                          // [kAlignWaves][E]
  int* seg_start = smem + kAlignWaves * E;     // [E + 1]
  int* scan_tmp = seg_start + (E + 1);         // [2 * kAlignWaves]

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  for (int i = tid; i < kAlignWaves * E; i += kAlignThreads) counts[i] = 0;
  __syncthreads();

  const int chunk = ((P + kAlignWaves - 1) / kAlignWaves + kWave - 1) / kWave * kWave;
  const int c0 = wave * chunk;
  const int c1 = min(P, c0 + chunk);

  // The wave's chunk is read in batches of kBatch ids per lane, all loads of
  // a batch in flight together (the loop is latency-bound otherwise).
  // pass 1: histogram of this wave's chunk
  for (int base = c0; base < c1; base += kWave * kBatch) {
    int ids[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base + j * kWave + lane;
      ids[j] = i < c1 ? topk_ids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (ids[j] >= 0 && ids[j] < E) atomicAdd(&counts[wave * E + ids[j]], 1);
  }
  __syncthreads();

  // per-expert exclusive prefix over waves, and padded segment sizes
  for (int e = tid; e < E; e += kAlignThreads) {
    int run = 0;
    for (int w = 0; w < kAlignWaves; ++w) {
      const int c = counts[w * E + e];
      counts[w * E + e] = run;
      run += c;
    }
    seg_start[e] = (run + B - 1) / B * B;   // padded size for now
  }
  __syncthreads();

  // exclusive scan of padded sizes over experts (E <= 1024 = one per thread):
  // inclusive scan inside each wave by shuffles, then over the wave totals.
  {
    const int v = (tid < E) ? seg_start[tid] : 0;
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) scan_tmp[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int w = lane < kAlignWaves ? scan_tmp[lane] : 0;
#pragma unroll
      for (int off = 1; off < kAlignWaves; off <<= 1) {
        const int y = __shfl_up(w, off, kWave);
        if (lane >= off) w += y;
      }
      if (lane < kAlignWaves) scan_tmp[kAlignWaves + lane] = w;   // inclusive wave totals
    }
    __syncthreads();
    const int before = wave ? scan_tmp[kAlignWaves + wave - 1] : 0;
    if (tid < E) seg_start[tid] = before + x - v;   // exclusive
    if (tid == 0) seg_start[E] = scan_tmp[2 * kAlignWaves - 1];
  }
  __syncthreads();
  const int total = seg_start[E];

  // pass 2: stable scatter
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = c0; base < c1; base += kWave * kBatch) {
    int ids[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base + j * kWave + lane;
      ids[j] = i < c1 ? topk_ids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = base + j * kWave + lane;
      const int e = ids[j];
      const bool ok = e >= 0 && e < E;
      uint64_t match = __ballot(ok);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = ok && ((e >> b) & 1);
        const uint64_t m = __ballot(bit);
        match &= bit ? m : ~m;
      }
      if (ok) {
        const int rank = __popcll(match & lt_mask);
        const int cur = counts[wave * E + e];
        sorted_ids[seg_start[e] + cur + rank] = i;
        // the highest lane of the group advances the cursor
        if ((match >> lane) == 1ull) counts[wave * E + e] = cur + __popcll(match);
      }
    }
  }

  // placeholders inside segments, expert id per block
  __syncthreads();
  for (int e = tid; e < E; e += kAlignThreads) {
    // after pass 2 the last wave's cursor for e equals the count of e
    const int cnt = counts[(kAlignWaves - 1) * E + e];
    const int s0 = seg_start[e], s1 = seg_start[e + 1];
    for (int s = s0 + cnt; s < s1; ++s) sorted_ids[s] = P;
    for (int blk = s0 / B; blk < s1 / B; ++blk) expert_ids[blk] = e;
  }
  for (int s = total + tid; s < max_padded; s += kAlignThreads) sorted_ids[s] = P;
  for (int blk = total / B + tid; blk < max_padded / B; blk += kAlignThreads) expert_ids[blk] = -1;
  if (tid == 0) *total_out = total;
}

// ---------------------------------------------------------------------------
// Expert-parallel variant: one workgroup per expert, for the common sizes.
//
// Every workgroup reads all the ids (a few hundred KiB at most, served from
// L2), builds the full per-expert histogram in LDS and scans the padded
// sizes itself, so no workgroup waits for another and nothing has to be
// staged in global memory.  Workgroup e then writes only expert e's segment:
// wave w owns the w-th contiguous run of pairs, counts its pairs of expert
// e, and a block-wide exclusive scan of those counts gives each wave where
// its pairs go.  Runs are in pair order and each run is written in order,
// so the segment is in ascending pair order (stable).  Placeholders, expert
// ids per block and the unused tail of both buffers are written alongside.
// The ids are cached in LDS as 16-bit values when they fit.
constexpr int kAlignEThreads = 512;
constexpr int kAlignEWaves = kAlignEThreads / kWave;
constexpr int kAlignEBatch = 64;   // ids per thread in flight at once (one round trip for 32K pairs)

// Exclusive scan of one int per thread over the workgroup; also returns the
// total.  tmp: LDS scratch of 2 * kAlignEWaves ints.  Contains barriers.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kAlignEWaves ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < kAlignEWaves; off <<= 1) {
      const int y = __shfl_up(w, off, kWave);
      if (lane >= off) w += y;
    }
    if (lane < kAlignEWaves) tmp[kAlignEWaves + lane] = w;
  }
  __syncthreads();
  total = tmp[2 * kAlignEWaves - 1];
  const int before = wave ? tmp[kAlignEWaves + wave - 1] : 0;
  __syncthreads();   // tmp may be reused right after
  return before + x - v;
}

template <bool CACHE>
__global__ void __launch_bounds__(kAlignEThreads)
align_expert_kernel(const int32_t* __restrict__ topk_ids, int P, int E, int B,
                    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ expert_ids,
                    int32_t* __restrict__ total_out, int max_padded) {
  extern __shared__ int smem[];
  int* hist = smem;                                  // [kAlignEWaves][E]
  int* seg = hist + kAlignEWaves * E;                // [E + 1] segment starts
  int* tmp = seg + (E + 1);                          // [2 * kAlignEWaves]
  uint16_t* cache = reinterpret_cast<uint16_t*>(tmp + 2 * kAlignEWaves);   // [P] if CACHE

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int e = blockIdx.x;
  for (int i = tid; i < kAlignEWaves * E; i += kAlignEThreads) hist[i] = 0;
  __syncthreads();

  // 1. histogram of all pairs (per-wave copies keep LDS atomics apart)
  for (int base = 0; base < P; base += kAlignEThreads * kAlignEBatch) {
    int ids[kAlignEBatch];
#pragma unroll
    for (int j = 0; j < kAlignEBatch; ++j) {
      const int i = base + j * kAlignEThreads + tid;
      ids[j] = i < P ? topk_ids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kAlignEBatch; ++j) {
      const int i = base + j * kAlignEThreads + tid;
      const bool ok = ids[j] >= 0 && ids[j] < E;
      if (ok) atomicAdd(&hist[wave * E + ids[j]], 1);
      if (CACHE && i < P) cache[i] = ok ? (uint16_t)ids[j] : (uint16_t)0xFFFFu;
    }
  }
  __syncthreads();

  // 2. padded segment sizes and their exclusive scan (two experts per thread)
  int cnt2[2] = {0, 0};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int ee = 2 * tid + q;
    if (ee < E)
      for (int w = 0; w < kAlignEWaves; ++w) cnt2[q] += hist[w * E + ee];
  }
  const int pad0 = (cnt2[0] + B - 1) / B * B, pad1 = (cnt2[1] + B - 1) / B * B;
  int total;
  const int start = block_exclusive_scan(pad0 + pad1, tmp, total);
  if (2 * tid < E) seg[2 * tid] = start;
  if (2 * tid + 1 < E) seg[2 * tid + 1] = start + pad0;
  if (tid == 0) seg[E] = total;
  __syncthreads();

  // 3. this expert's pairs, stable: wave w walks the w-th contiguous run of
  //    pairs 64 at a time (consecutive lanes read consecutive ids), counts
  //    its matches, and after a scan over the waves writes them, each lane
  //    at the wave's cursor plus its rank among the matching lanes.
  const int run = (P + kAlignEWaves * kWave - 1) / (kAlignEWaves * kWave) * kWave;
  const int r0 = min(P, wave * run), r1 = min(P, r0 + run);
  auto id_at = [&](int i) -> int { return CACHE ? (int)cache[i] : topk_ids[i]; };
  int mine = 0;
#pragma unroll 8
  for (int i = r0 + lane; i < r1; i += kWave) mine += id_at(i) == e;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mine += __shfl_xor(mine, m, kWave);
  int cnt_e;
  int cursor = seg[e] + block_exclusive_scan(lane == 0 ? mine : 0, tmp, cnt_e);
  cursor = __shfl(cursor, 0, kWave);
  if (mine) {
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int base = r0; base < r1; base += kWave) {
      const int i = base + lane;
      const bool hit = i < r1 && id_at(i) == e;
      const uint64_t m = __ballot(hit);
      if (hit) sorted_ids[cursor + __popcll(m & lt_mask)] = i;
      cursor += __popcll(m);
    }
  }

  // 4. placeholders and expert ids of this segment
  const int s0 = seg[e], s1 = seg[e + 1];
  for (int s = s0 + cnt_e + tid; s < s1; s += kAlignEThreads) sorted_ids[s] = P;
  for (int b = s0 / B + tid; b < s1 / B; b += kAlignEThreads) expert_ids[b] = e;

  // 5. unused tail of both buffers, shared by all workgroups
  const int stride = gridDim.x * kAlignEThreads, first = blockIdx.x * kAlignEThreads + tid;
  for (int s = total + first; s < max_padded; s += stride) sorted_ids[s] = P;
  for (int b = total / B + first; b < max_padded / B; b += stride) expert_ids[b] = -1;
  if (blockIdx.x == 0 && tid == 0) *total_out = total;
}

// ---------------------------------------------------------------------------
// Two-kernel variant with a workspace (moe_forward).  The pairs are cut into
// chunks of `chunk` ids, one workgroup each.
//   count: per-chunk histogram hist[c][e] into the workspace;
//   place: every chunk reads all counts, scans the padded segment sizes, and
//          places its own pairs: expert e's pairs of chunk c start at
//          seg[e] + (pairs of e in chunks before c); inside the chunk each wave
//          owns a contiguous run and ranks matching lanes with one ballot per
//          bit of the expert id, so segments stay in ascending pair order.
//          Placeholders, expert ids per block and the unused tail are split
//          over the chunks.
constexpr int kCountThreads = 256;
constexpr int kPlaceThreads = 512;
constexpr int kPlaceWaves = kPlaceThreads / kWave;
constexpr int64_t kAlignSelfPairs = 2048;   // one chunk of the two-kernel path

__global__ void __launch_bounds__(kCountThreads)
align_count_kernel(const int32_t* __restrict__ topk_ids, int P, int E, int chunk,
                   int32_t* __restrict__ hist) {
  extern __shared__ int cnt[];
  for (int e = threadIdx.x; e < E; e += kCountThreads) cnt[e] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * chunk, c1 = min(P, c0 + chunk);
  constexpr int kB = 8;   // ids per thread in flight at once
  for (int base = c0; base < c1; base += kB * kCountThreads) {
    int v[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int i = base + j * kCountThreads + (int)threadIdx.x;
      v[j] = i < c1 ? topk_ids[i] : -1;
    }
#pragma unroll
    for (int j = 0; j < kB; ++j)
      if (v[j] >= 0 && v[j] < E) atomicAdd(&cnt[v[j]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kCountThreads) hist[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan of one int per thread over a kPlaceThreads workgroup.
__device__ __forceinline__ int place_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kPlaceWaves ? tmp[lane] : 0;
#pragma unroll
    for (int off = 1; off < kPlaceWaves; off <<= 1) {
      const int y = __shfl_up(w, off, kWave);
      if (lane >= off) w += y;
    }
    if (lane < kPlaceWaves) tmp[kPlaceWaves + lane] = w;
  }
  __syncthreads();
  total = tmp[2 * kPlaceWaves - 1];
  const int before = wave ? tmp[kPlaceWaves + wave - 1] : 0;
  __syncthreads();
  return before + x - v;
}

// SELF: one workgroup takes every pair (c = 0, chunk = P) and counts the
// experts itself from its per-wave counts, without a count kernel's
// histogram (hist is not read).
template <bool SELF>
__global__ void __launch_bounds__(kPlaceThreads)
align_place_kernel(const int32_t* __restrict__ topk_ids, int P, int E, int B, int chunk, int nchunk,
                   const int32_t* __restrict__ hist, int32_t* __restrict__ sorted_ids,
                   int32_t* __restrict__ expert_ids, int32_t* __restrict__ total_out,
                   int max_padded, int32_t* __restrict__ wide_table) {
  extern __shared__ int smem[];
  int* seg = smem;                               // [E + 1] segment starts
  int* cur = seg + (E + 1);                      // [kPlaceWaves][E] per-wave cursors
  int* tot = cur + kPlaceWaves * E;              // [E] pairs per expert
  int* tmp = tot + E;                            // [2 * kPlaceWaves]
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int c = blockIdx.x;

  // this wave's run of the chunk, read once into registers kR ids per lane
  // at a time when it is short
  const int c0 = c * chunk, c1 = min(P, c0 + chunk);
  const int run = (chunk + kPlaceWaves * kWave - 1) / (kPlaceWaves * kWave) * kWave;
  const int r0 = min(c1, c0 + wave * run), r1 = min(c1, r0 + run);
  constexpr int kR = 4;
  const bool one_batch = r1 - r0 <= kR * kWave;
  int v[kR];
  // per-wave counts of this chunk
  auto count_runs = [&]() {
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int i = r0 + j * kWave + lane;
      v[j] = i < r1 ? topk_ids[i] : -1;
    }
    if (one_batch) {
#pragma unroll
      for (int j = 0; j < kR; ++j)
        if (v[j] >= 0 && v[j] < E) atomicAdd(&cur[wave * E + v[j]], 1);
    } else {
      for (int i = r0 + lane; i < r1; i += kWave) {
        const int e = topk_ids[i];
        if (e >= 0 && e < E) atomicAdd(&cur[wave * E + e], 1);
      }
    }
  };

  // totals, and pairs of each expert in the chunks before this one
  int padded[2] = {0, 0}, before_c[2] = {0, 0};
  if constexpr (SELF) {
    for (int i = tid; i < kPlaceWaves * E; i += kPlaceThreads) cur[i] = 0;
    __syncthreads();
    count_runs();
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = 2 * tid + q;
      if (e < E) {
        int t = 0;
        for (int w = 0; w < kPlaceWaves; ++w) t += cur[w * E + e];
        tot[e] = t;
        padded[q] = (t + B - 1) / B * B;
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = 2 * tid + q;
      if (e < E) {
        int t = 0, b = 0;
#pragma unroll 16
        for (int cc = 0; cc < nchunk; ++cc) {   // independent loads, issued together
          const int h = hist[(int64_t)cc * E + e];
          t += h;
          b += cc < c ? h : 0;
        }
        tot[e] = t;
        padded[q] = (t + B - 1) / B * B;
        before_c[q] = b;
      }
    }
  }
  int total;
  const int start = place_exclusive_scan(padded[0] + padded[1], tmp, total);
  if (2 * tid < E) seg[2 * tid] = start;
  if (2 * tid + 1 < E) seg[2 * tid + 1] = start + padded[0];
  if (tid == 0) seg[E] = total;
  if constexpr (!SELF)
    for (int i = tid; i < kPlaceWaves * E; i += kPlaceThreads) cur[i] = 0;
  __syncthreads();

  // The first chunk also writes the expert-wide tile table: each expert's
  // blocks in ceil(n / kWideMaxBlocks) runs of near-equal length.
  if (wide_table && c == 0) {
    int nb[2], nt[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      nb[q] = padded[q] / B;
      nt[q] = (nb[q] + kWideMaxBlocks - 1) / kWideMaxBlocks;
    }
    int ntiles;
    int j = place_exclusive_scan(nt[0] + nt[1], tmp, ntiles);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int e = 2 * tid + q;
      if (e < E) {
        const int first = seg[e] / B;
        for (int i = 0; i < nt[q]; ++i, ++j) {
          const int b0 = first + (int)((int64_t)i * nb[q] / nt[q]);
          const int b1 = first + (int)((int64_t)(i + 1) * nb[q] / nt[q]);
          wide_table[1 + 3 * j] = e;
          wide_table[2 + 3 * j] = b0;
          wide_table[3 + 3 * j] = b1 - b0;
        }
      }
    }
    if (tid == 0) wide_table[0] = ntiles;
  }

  // per-wave counts of this chunk (already taken in SELF mode), then each
  // wave's first slot per expert
  if constexpr (!SELF) {
    count_runs();
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * tid + q;
    if (e < E) {
      int run_e = seg[e] + before_c[q];
      for (int w = 0; w < kPlaceWaves; ++w) {
        const int n = cur[w * E + e];
        cur[w * E + e] = run_e;
        run_e += n;
      }
    }
  }
  __syncthreads();

  // stable scatter: lanes with the same expert find each other by ballots
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  for (int base = r0, j = 0; base < r1; base += kWave, ++j) {
    const int i = base + lane;
    int e;
    if (one_batch) {   // j < kR here
      e = v[0];
#pragma unroll
      for (int q = 1; q < kR; ++q) e = j == q ? v[q] : e;
    } else {
      e = i < r1 ? topk_ids[i] : -1;
    }
    const bool ok = e >= 0 && e < E;
    uint64_t match = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    if (ok) {
      const int pos = cur[wave * E + e];
      sorted_ids[pos + __popcll(match & lt_mask)] = i;
      if ((match >> lane) == 1ull) cur[wave * E + e] = pos + __popcll(match);   // highest lane
    }
  }

  // Placeholders: the padding slots (fewer than B) of the experts
  // e = c, c + nchunk, ..., flattened over (expert, slot) so that no thread
  // walks the experts one after another.
  const int nloc = c < E ? (E - c + nchunk - 1) / nchunk : 0;
  for (int i = tid; i < nloc * B; i += kPlaceThreads) {
    const int e = c + (i / B) * nchunk, s = i % B;
    const int p = seg[e] + tot[e] + s;
    if (p < seg[e + 1]) sorted_ids[p] = P;
  }
  // Expert of each used block, blocks split over the chunks: the last
  // expert whose segment starts at or before the block (that segment is not
  // empty and holds the block).
  const int stride = nchunk * kPlaceThreads, first = c * kPlaceThreads + tid;
  for (int b = first; b < total / B; b += stride) {
    const int pos = b * B;
    int lo = 0, hi = E;   // seg[lo] <= pos < seg[hi] (seg[E] = total)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seg[mid] <= pos) lo = mid; else hi = mid;
    }
    expert_ids[b] = lo;
  }
  for (int s = total + first; s < max_padded; s += stride) sorted_ids[s] = P;
  for (int b = total / B + first; b < max_padded / B; b += stride) expert_ids[b] = -1;
  if (c == 0 && tid == 0) *total_out = total;
}

int64_t align_ws_chunk(int64_t P) {
  const int64_t c = (P + 1023) / 1024;   // at most 1024 chunks
  return c < 2048 ? 2048 : c;
}

size_t align_ws_bytes(int64_t P, int E) {
  const int64_t chunk = align_ws_chunk(P);
  const int64_t n = P > 0 ? (P + chunk - 1) / chunk : 1;
  return sizeof(int32_t) * (size_t)n * (size_t)E;
}

hipError_t launch_align_ws(const int32_t* topk_ids, int64_t P, int E, int B, int32_t* sorted_ids,
                           int32_t* expert_ids, int32_t* total, int64_t max_padded, int32_t* hist,
                           hipStream_t stream, int32_t* wide_table) {
  if (wide_table && (B != kWideBlockRows || E > kWidePrepMaxExperts || E > 2 * kPlaceThreads))
    return hipErrorInvalidValue;
  // Up to kAlignSelfPairs pairs one workgroup counts and places them all;
  // beyond, per-chunk counts first, then placement by every chunk.
  const bool self = P <= kAlignSelfPairs;
  const int64_t chunk = self ? (P > 0 ? P : 1) : align_ws_chunk(P);
  const int nchunk = P > 0 ? (int)((P + chunk - 1) / chunk) : 1;
  hipError_t st;
  if (!self) {
    hipLaunchKernelGGL(align_count_kernel, dim3(nchunk), dim3(kCountThreads), sizeof(int) * E,
                       stream, topk_ids, (int)P, E, (int)chunk, hist);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
  }
  void (*place)(const int32_t*, int, int, int, int, int, const int32_t*, int32_t*, int32_t*,
                int32_t*, int, int32_t*) =
      self ? align_place_kernel<true> : align_place_kernel<false>;
  const size_t lds = sizeof(int) * ((size_t)(E + 1) + (size_t)kPlaceWaves * E + E + 2 * kPlaceWaves);
  st = raise_lds_limit(reinterpret_cast<const void*>(place), lds);
  if (st != hipSuccess) return st;
  hipLaunchKernelGGL(place, dim3(nchunk), dim3(kPlaceThreads), lds, stream, topk_ids,
                     (int)P, E, B, (int)chunk, nchunk, hist, sorted_ids, expert_ids, total,
                     (int)max_padded, wide_table);
  return hipGetLastError();
}

hipError_t launch_align(const int32_t* topk_ids, int64_t P, int E, int B,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* total,
                        int64_t max_padded, hipStream_t stream) {
  // Expert-parallel kernel while every workgroup's full read of the ids stays
  // cheap; the single-workgroup kernel beyond that.
  if (P * (int64_t)E <= ((int64_t)1 << 26)) {
    const size_t base = sizeof(int) * ((size_t)kAlignEWaves * E + (E + 1) + 2 * kAlignEWaves);
    const size_t with_cache = base + 2 * (size_t)P;
    const bool cache = with_cache <= 160 * 1024;
    const size_t lds = cache ? with_cache : base;
    auto k = cache ? align_expert_kernel<true> : align_expert_kernel<false>;
    const hipError_t st = raise_lds_limit(reinterpret_cast<const void*>(k), lds);
    if (st != hipSuccess) return st;
    hipLaunchKernelGGL(k, dim3(E), dim3(kAlignEThreads), lds, stream, topk_ids, (int)P, E, B,
                       sorted_ids, expert_ids, total, (int)max_padded);
    return hipGetLastError();
  }
  const size_t lds = sizeof(int) * ((size_t)kAlignWaves * E + (E + 1) + 2 * kAlignWaves);
  {
    const hipError_t st = raise_lds_limit(reinterpret_cast<const void*>(align_kernel), lds);
    if (st != hipSuccess) return st;
  }
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), lds, stream, topk_ids,
                     (int)P, E, B, sorted_ids, expert_ids, total, (int)max_padded);
  return hipGetLastError();
}

}  // namespace moe

// Alignment kernel: stable sort of (token, expert) pairs by expert with every
// expert's segment padded to a multiple of block_m.
//
// Semantics: mini-sglang "MoE and fused MoE", moe_align_block_size (stable
// argsort by expert, placeholder = number of pairs, one expert id per block).
//
// Design: a single 1024-thread workgroup (16 waves); totals never leave the
// device.  Wave w owns a contiguous chunk of the pairs.
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

hipError_t launch_align(const int32_t* topk_ids, int64_t P, int E, int B,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* total,
                        int64_t max_padded, hipStream_t stream) {
  const size_t lds = sizeof(int) * ((size_t)kAlignWaves * E + (E + 1) + 2 * kAlignWaves);
  if (lds > 65536) {
    const hipError_t st = hipFuncSetAttribute(
        (const void*)align_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (st != hipSuccess) return st;
  }
  hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kAlignThreads), lds, stream, topk_ids,
                     (int)P, E, B, sorted_ids, expert_ids, total, (int)max_padded);
  return hipGetLastError();
}

}  // namespace moe

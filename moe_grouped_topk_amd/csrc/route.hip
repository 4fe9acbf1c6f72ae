// Routing kernel: GroupedTopK / plain top-k with softmax or sigmoid scores.
//
// Semantics: "GroupedTopK operator optimisation primer", sections 三 3.1-3.6
// (scores, group max, top groups, mask, top-k, renormalise and scale); plain
// top-k (mini-sglang "MoE and fused MoE", select_experts) is one group.
//
// Design: one 64-lane wavefront per token, everything in registers.  Lane l
// holds experts [l*V, l*V + V).  Selection works on order-preserving integer
// keys of the LOGITS: both scorings are monotone, so the order of the logits
// is the order of the exact scores (the primer's section 七 shortcut), and
// no rounding of exp() can merge or swap two candidates.  A candidate is the
// 64-bit value (key << 32) | (0xffffffff - index): its maximum is the largest
// logit with the lowest index among equals.  Each top-k round is a lane-local
// max over V values plus a 6-step xor-shuffle max across the wave (group
// stage); the final top-k is a radix select on the keys with ballots.
// Weights (softmax + renormalise) are a softmax over the k selected logits
// alone, since the full-row denominator cancels (section 七); the other
// variants keep the full denominator or use the sigmoid scores.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

// QX (int8 layer): 0 none; 1 / 2: the token's row of bf16 / f32 x is also
// quantised per row (low-precision GMM article, section 3.2: the scale is
// taken from the row as it is loaded), and ex.zero is cleared.
template <int V, int QX>
__global__ void __launch_bounds__(256)
route_kernel(const float* __restrict__ gating, int64_t T, int E, int topk,
             int G, int topk_group, int scoring, int renormalize, float scale,
             float* __restrict__ out_w, int32_t* __restrict__ out_ids, RouteExtra ex) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if constexpr (QX != 0) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ex.nzero;
         i += (int64_t)gridDim.x * blockDim.x)
      ex.zero[i] = 0;
  }
  if (t >= T) return;
  const float* row = gating + t * (int64_t)E;

  float x[V];
  uint64_t cand[V];
  const int e0 = lane * V;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = e0 + j;
    x[j] = (e < E) ? row[e] : 0.0f;
    cand[j] = (e < E) ? (((uint64_t)float_key(x[j]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e))
                      : 0ull;
  }

  // Group stage ([GTK] 3.2-3.4): group score = max logit of the group; keep
  // the topk_group best groups (ties -> lower group), mask the others.
  const int P = G > 1 ? E / G : E;
  const int seg = P / V;   // lanes per group when a group is a whole number of lanes
  if (G > 1 && G <= kWave && P % V == 0 && (seg & (seg - 1)) == 0) {
    // Each group is an aligned run of seg lanes: its max by seg-lane xor
    // steps, all groups at once; then every group's rank among the G group
    // maxima (ties to the lower group) from the maxima read lane by lane.
    uint32_t m = 0u;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const uint32_t k = (uint32_t)(cand[j] >> 32);
      m = k > m ? k : m;
    }
    for (int st = 1; st < seg; st <<= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)m, st, kWave);
      m = o > m ? o : m;
    }
    const int my_g = lane / seg;
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      const uint32_t mg = (uint32_t)__builtin_amdgcn_readlane((int)m, g * seg);
      rank += (mg > m || (mg == m && g < my_g)) ? 1 : 0;
    }
    if (rank >= topk_group) {
#pragma unroll
      for (int j = 0; j < V; ++j) cand[j] = 0ull;
    }
  } else if (G > 1) {
    uint64_t gcand = 0ull;   // lane g < G holds group g's candidate
    for (int g = 0; g < G; ++g) {
      uint32_t m = 0u;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int e = e0 + j;
        if (e < E && e / P == g) {
          const uint32_t k = (uint32_t)(cand[j] >> 32);
          m = k > m ? k : m;
        }
      }
      m = wave_max_u32(m);
      if (lane == g) gcand = ((uint64_t)m << 32) | (uint64_t)(0xffffffffu - (uint32_t)g);
    }
    uint64_t kept = 0ull;    // bit g set: group g kept
    for (int r = 0; r < topk_group; ++r) {
      const uint64_t best = wave_max_u64(gcand);
      const int g = (int)(0xffffffffu - (uint32_t)best);
      kept |= 1ull << g;
      if (lane == g) gcand = 0ull;
    }
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int e = e0 + j;
      if (e < E && !((kept >> (e / P)) & 1ull)) cand[j] = 0ull;
    }
  }

  // Top-k ([GTK] 3.5, 八), by a radix select on the 32-bit keys: bit by bit
  // from the top, keep the largest threshold th with at least topk keys >= th
  // (ballot counts, no cross-lane data movement).  The picks are the keys
  // above th plus, among the keys equal to th, the lowest indices.  Masked
  // and absent experts hold key 0, which no finite or -inf logit reaches.
  uint32_t key[V];
#pragma unroll
  for (int j = 0; j < V; ++j) key[j] = (uint32_t)(cand[j] >> 32);
  uint32_t th = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = th | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < V; ++j) n += __popcll(__ballot(key[j] >= c));
    if (n >= topk) th = c;
  }
  // keys strictly above th are all picked; ties at th fill the rest in index
  // order (expert e = lane * V + j, so index order is lane order, then j)
  int above = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) above += __popcll(__ballot(key[j] > th));
  int need = topk - above;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  bool pick[V];
  uint64_t tie_before = 0;   // ties at th in lanes below this one (all j)
#pragma unroll
  for (int j = 0; j < V; ++j) tie_before += __popcll(__ballot(key[j] == th) & lt_mask);
  int rank_tie = (int)tie_before;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const bool tie = key[j] == th && key[j] != 0u;
    pick[j] = key[j] > th || (tie && rank_tie < need);
    if (key[j] == th) ++rank_tie;
  }
  // Order the picks (key descending, index ascending): the rank of a pick is
  // the number of picks ahead of it.  Picks are gathered into lanes 0..topk-1
  // by their position in index order, then each compares against the others.
  int before = 0;
#pragma unroll
  for (int j = 0; j < V; ++j) before += __popcll(__ballot(pick[j]) & lt_mask);
  __shared__ uint64_t s_pick[4][kWave];
  const int wslot = (threadIdx.x / kWave) & 3;
  int q = before;
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (pick[j]) s_pick[wslot][q++] = cand[j];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const uint64_t mine_c = lane < topk ? s_pick[wslot][lane] : 0ull;
  int rank = 0;
  for (int r = 0; r < topk; ++r) rank += s_pick[wslot][r] > mine_c;
  // lane r must end up with the r-th pick: move through LDS once more
  __builtin_amdgcn_wave_barrier();
  if (lane < topk) s_pick[wslot][rank] = mine_c;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  const uint64_t my_c = lane < topk ? s_pick[wslot][lane] : 0ull;
  const int my_id = (int)(0xffffffffu - (uint32_t)my_c);
  const float my_x = key_float((uint32_t)(my_c >> 32));
  // the first pick is the row's largest logit: the best expert's group is kept
  const float top_x = key_float((uint32_t)(s_pick[wslot][0] >> 32));

  // Weights ([GTK] 3.1 and 3.6).
  float w;
  const bool mine = lane < topk;
  if (scoring == 0) {
    // top_x is the row maximum: the best group holds the best expert.
    const float ek = mine ? expf(my_x - top_x) : 0.0f;
    float den;
    if (renormalize) {
      den = wave_sum_f32(ek);
    } else {
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (e0 + j < E) s += expf(x[j] - top_x);
      den = wave_sum_f32(s);
    }
    w = ek / den;
  } else {
    const float sk = mine ? 1.0f / (1.0f + expf(-my_x)) : 0.0f;
    if (renormalize) {
      const float den = wave_sum_f32(sk);
      w = sk / den;
    } else {
      w = sk;
    }
  }
  w *= scale;
  if (mine) {
    out_w[t * topk + lane] = w;
    out_ids[t * topk + lane] = my_id;
  }
  if constexpr (QX != 0) {
    // max |x| of the row (wave max), then its codes, 8 values per lane per step
    constexpr int XDT = QX == 1 ? 1 : 0;
    const void* xr = reinterpret_cast<const uint8_t*>(ex.x) + t * ex.cols * (XDT == 1 ? 2 : 4);
    float amax = 0.0f;
    for (int64_t i = (int64_t)lane * 8; i < ex.cols; i += kWave * 8) {
      float v[8];
      load8<XDT>(xr, i, v);
#pragma unroll
      for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kWave));
    const float qs = quant_scale(amax);
    int8_t* qr = ex.q + t * ex.cols;
    for (int64_t i = (int64_t)lane * 8; i < ex.cols; i += kWave * 8) {
      float v[8];
      load8<XDT>(xr, i, v);
      *reinterpret_cast<uint2*>(qr + i) = make_uint2(code4(v, qs), code4(v + 4, qs));
    }
    if (lane == 0) ex.scales[t] = qs;
  }
}

hipError_t launch_route(const float* gating, int64_t T, int E, int topk, int G,
                        int topk_group, int scoring, int renormalize, float scale,
                        float* out_w, int32_t* out_ids, hipStream_t stream,
                        const RouteExtra* extra) {
  if (T == 0) return hipSuccess;
  const int waves_per_block = 4;
  const dim3 block(kWave * waves_per_block);
  const dim3 grid((unsigned)((T + waves_per_block - 1) / waves_per_block));
  const int per_lane = (E + kWave - 1) / kWave;
  const RouteExtra ex = extra ? *extra : RouteExtra{};
  const int qx = extra ? (extra->x_dtype == 1 ? 1 : 2) : 0;
#define MOE_ROUTE_LAUNCH(VV, QQ)                                                        \
  hipLaunchKernelGGL((route_kernel<VV, QQ>), grid, block, 0, stream, gating, T, E, topk, \
                     G, topk_group, scoring, renormalize, scale, out_w, out_ids, ex)
#define MOE_ROUTE_CASE(VV)                  \
  do {                                      \
    if (qx == 0) MOE_ROUTE_LAUNCH(VV, 0);   \
    else if (qx == 1) MOE_ROUTE_LAUNCH(VV, 1); \
    else MOE_ROUTE_LAUNCH(VV, 2);           \
  } while (0)
  if (per_lane <= 1) MOE_ROUTE_CASE(1);
  else if (per_lane <= 2) MOE_ROUTE_CASE(2);
  else if (per_lane <= 4) MOE_ROUTE_CASE(4);
  else if (per_lane <= 8) MOE_ROUTE_CASE(8);
  else MOE_ROUTE_CASE(16);
#undef MOE_ROUTE_CASE
#undef MOE_ROUTE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe

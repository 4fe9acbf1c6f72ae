// One-time re-layout of expert weights into the packed tile layout of
// moe_pack_weights (moe.h): per (expert, 256-row tile, 64-byte K stage) one
// contiguous 16 KiB block holding exactly the swizzled LDS image the tile
// kernels stage, so their K loop reads HBM contiguously.

#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// One thread per 16-byte output chunk (grid-stride).  Reads are 16-byte
// chunks of the plain rows, writes are fully coalesced.
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* w, int64_t N, int64_t kbytes,
                                                  int silu, int64_t NT, int64_t KS,
                                                  int64_t nchunks, uint8_t* out) {
  const u32x4_t zero = {0u, 0u, 0u, 0u};
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < nchunks;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t blk = u / (kPackBlockBytes / 16);
    const int within = (int)(u % (kPackBlockBytes / 16));
    const int r = within / 4, pos = within % 4;
    const int64_t ks = blk % KS, t = (blk / KS) % NT, e = blk / (KS * NT);
    const int c = pos ^ ((r >> 2) & 3);                  // chunk stored at this position
    const int64_t kb = ks * kPackStageBytes + c * 16;    // byte offset inside the row
    int64_t row;
    bool ok;
    if (silu) {
      const int64_t half = N / 2, col = t * (kPackRows / 2) + (r % (kPackRows / 2));
      ok = col < half;
      row = r < kPackRows / 2 ? col : half + col;
    } else {
      row = t * kPackRows + r;
      ok = row < N;
    }
    u32x4_t v = zero;
    if (ok && kb < kbytes)
      v = *reinterpret_cast<const u32x4_t*>(w + (e * N + row) * kbytes + kb);
    *reinterpret_cast<u32x4_t*>(out + u * 16) = v;
  }
}

}  // namespace

hipError_t launch_pack_weights(const void* w, int elem_bytes, int E, int64_t N, int64_t K, int silu,
                               void* packed, hipStream_t stream) {
  const int64_t NT = packed_tiles(N, silu), KS = packed_kstages(K, elem_bytes);
  const int64_t nchunks = (int64_t)E * NT * KS * (kPackBlockBytes / 16);
  if (nchunks == 0) return hipSuccess;
  const int64_t want = (nchunks + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(w), N, K * elem_bytes, silu, NT, KS, nchunks,
                     reinterpret_cast<uint8_t*>(packed));
  return hipGetLastError();
}

}  // namespace moe

// Block copies between pools: the copy of copy-on-write inside one pool, and
// swap-in / swap-out between a GPU pool and a pinned host pool.
//
// Copy-on-write: a write into a block that other sequences still reference
// (reference count 2 or more) goes to a copy of it (SOSP 2023 PagedAttention
// explainer, "Copy-on-Writeによるメモリ共有").  Swap: KV evicted from the GPU
// lives in a CPU tier of blocks, and comes back one layer at a time, the next
// layer's transfer overlapping this layer's attention (Pensieve explainer,
// "GPU-CPU 2層キャッシュ構造", "パイプライン化されたswap-in").  16-token
// blocks are too small a unit for separate host transfers (KV-cache textbook
// ch.14): here one launch moves a whole list of scattered blocks, reading
// each tile where it lies (device or host memory) and writing it where it
// goes, so no staging buffer and no per-block call.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// The copies' (block, KV head, K or V) tiles of 4 KiB, numbered block-major
// (K of every head of a block, then its V), are spread over a bounded grid:
// each of at most kCopyWorkgroups workgroups takes kTilesInFlight
// consecutive tiles per round, every lane loading its 16-B vector of each
// before storing any, so each lane keeps that many loads in flight.  The
// grid stays small whatever the list's length: the copy leaves most of the
// chip's wave slots to kernels running beside it (an attention kernel whose
// grid is sized to be resident at once, during a pipelined swap-in), and
// across the host link it is the loads in flight, not the workgroups, that
// carry the bandwidth.  Sources are read once: nontemporal.
constexpr int kCopyWorkgroups = 256;
constexpr int kTilesInFlight = 4;

__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ dst_k,
                                                          u32x4* __restrict__ dst_v,
                                                          const u32x4* __restrict__ src_k,
                                                          const u32x4* __restrict__ src_v,
                                                          const int32_t* __restrict__ src_ids,
                                                          const int32_t* __restrict__ dst_ids,
                                                          int32_t num_copies, int32_t src_blocks,
                                                          int32_t dst_blocks,
                                                          int32_t num_kv_heads) {
  constexpr int32_t kTileVecs = kBlockSize * kHeadDim * 2 / 16;  // 256 vectors of 16 B
  const uint32_t per_copy = 2u * (uint32_t)num_kv_heads;
  const uint32_t tiles = (uint32_t)num_copies * per_copy;
  const size_t per_block = (size_t)num_kv_heads * kTileVecs;
  for (uint32_t t0 = blockIdx.x * kTilesInFlight; t0 < tiles;
       t0 += gridDim.x * kTilesInFlight) {
    u32x4 v[kTilesInFlight];
    u32x4* to[kTilesInFlight];
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u) {
      to[u] = nullptr;
      const uint32_t t = t0 + u;  // uniform across the workgroup
      if (t >= tiles) continue;
      const uint32_t c = t / per_copy, r = t - c * per_copy;
      const bool is_v = r >= (uint32_t)num_kv_heads;
      const uint32_t h = is_v ? r - num_kv_heads : r;
      // A missing id list means block c of that pool (a staging run in order).
      const int32_t s = src_ids ? __builtin_amdgcn_readfirstlane(src_ids[c]) : (int32_t)c;
      const int32_t d = dst_ids ? __builtin_amdgcn_readfirstlane(dst_ids[c]) : (int32_t)c;
      if ((uint32_t)s >= (uint32_t)src_blocks || (uint32_t)d >= (uint32_t)dst_blocks) continue;
      const size_t lane = (size_t)h * kTileVecs + threadIdx.x;
      v[u] = load16_nt((is_v ? src_v : src_k) + (size_t)s * per_block + lane);
      to[u] = (is_v ? dst_v : dst_k) + (size_t)d * per_block + lane;
    }
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u)
      if (to[u]) *to[u] = v[u];
  }
}

hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* src_ids, const int32_t* dst_ids, int32_t num_copies,
                              int32_t src_blocks, int32_t dst_blocks, int32_t num_kv_heads,
                              hipStream_t stream) {
  if (num_copies == 0) return hipSuccess;
  const int64_t tiles = (int64_t)num_copies * 2 * num_kv_heads;
  const int64_t rounds = (tiles + kTilesInFlight - 1) / kTilesInFlight;
  const unsigned grid = (unsigned)(rounds < kCopyWorkgroups ? rounds : kCopyWorkgroups);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<u32x4*>(dst_k), static_cast<u32x4*>(dst_v),
                     static_cast<const u32x4*>(src_k), static_cast<const u32x4*>(src_v), src_ids,
                     dst_ids, num_copies, src_blocks, dst_blocks, num_kv_heads);
  return hipGetLastError();
}

}  // namespace pa

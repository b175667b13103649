// pa_copy_blocks: the block copy of copy-on-write.  A write into a block that
// other sequences still reference (reference count 2 or more) goes to a copy
// of it (SOSP 2023 PagedAttention explainer, "Copy-on-Writeによるメモリ共有");
// the host block manager picks the destination block, this kernel copies
// every KV head's K and V rows of the block, bit for bit.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// Workgroup (copy c, KV head h, tensor z): one (block, head) tile is 4 KiB =
// 256 vectors of 16 B, one per lane, so the read and the write are both one
// contiguous 4 KiB run.  The source is read once: nontemporal.
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ k_pool,
                                                          u32x4* __restrict__ v_pool,
                                                          const int32_t* __restrict__ src,
                                                          const int32_t* __restrict__ dst,
                                                          int32_t num_blocks,
                                                          int32_t num_kv_heads) {
  const int32_t s = src[blockIdx.x], d = dst[blockIdx.x];
  if ((uint32_t)s >= (uint32_t)num_blocks || (uint32_t)d >= (uint32_t)num_blocks) return;
  u32x4* pool = blockIdx.z == 0 ? k_pool : v_pool;
  constexpr int32_t kTileVecs = kBlockSize * kHeadDim * 2 / 16;  // 256
  const size_t head = (size_t)blockIdx.y * kTileVecs + threadIdx.x;
  const size_t per_block = (size_t)num_kv_heads * kTileVecs;
  pool[(size_t)d * per_block + head] = load16_nt(pool + (size_t)s * per_block + head);
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* src,
                              const int32_t* dst, int32_t num_copies, int32_t num_blocks,
                              int32_t num_kv_heads, hipStream_t stream) {
  if (num_copies == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_copies, num_kv_heads, 2), dim3(256), 0, stream,
                     static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), src, dst,
                     num_blocks, num_kv_heads);
  return hipGetLastError();
}

}  // namespace pa

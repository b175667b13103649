// pa_kv_write: scatter each new token's K and V rows into its pool slot.
//
// A new token goes into the slot its sequence appends to: the current block
// while it has room, else a freshly allocated block (SOSP 2023 PagedAttention
// explainer, "ブロックテーブルによるメモリ管理").  The caller resolves that to a
// slot = block * 16 + offset; -1 skips the token.  Pure data movement: every
// lane moves 16-byte vectors, so the copy is bit-exact for fp16 and bf16.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// One workgroup per token.  A (token, head) row is 256 B = 16 vectors of 16 B;
// the K rows of all heads come first, then the V rows.  Consecutive lanes take
// consecutive vectors, so both the read of k_new and the write into the
// (block, head, offset) row of the pool are contiguous 256-B runs.
__global__ __launch_bounds__(256) void kv_write_kernel(const u32x4* __restrict__ k_new,
                                                       const u32x4* __restrict__ v_new,
                                                       u32x4* __restrict__ k_pool,
                                                       u32x4* __restrict__ v_pool,
                                                       const int32_t* __restrict__ slot_mapping,
                                                       int32_t num_kv_heads) {
  const int32_t t = blockIdx.x;
  const int32_t slot = slot_mapping[t];
  if (slot < 0) return;
  const size_t block = (size_t)(slot >> 4);
  const int32_t offset = slot & 15;
  const int32_t per_tensor = num_kv_heads * 16;
  for (int32_t idx = threadIdx.x; idx < 2 * per_tensor; idx += blockDim.x) {
    const bool is_v = idx >= per_tensor;
    const int32_t rem = is_v ? idx - per_tensor : idx;
    const int32_t h = rem >> 4;
    const int32_t c = rem & 15;
    const size_t src = ((size_t)t * num_kv_heads + h) * 16 + c;
    const size_t dst = ((block * num_kv_heads + h) * kBlockSize + offset) * 16 + c;
    if (is_v)
      v_pool[dst] = v_new[src];
    else
      k_pool[dst] = k_new[src];
  }
}

hipError_t launch_kv_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = num_kv_heads * 32 >= 256 ? 256 : ((num_kv_heads * 32 + 63) / 64) * 64;
  hipLaunchKernelGGL(kv_write_kernel, dim3(num_tokens), dim3(threads), 0, stream,
                     static_cast<const u32x4*>(k_new), static_cast<const u32x4*>(v_new),
                     static_cast<u32x4*>(k_pool), static_cast<u32x4*>(v_pool), slot_mapping,
                     num_kv_heads);
  return hipGetLastError();
}

}  // namespace pa

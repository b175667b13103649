// Host-side launchers of the libpa kernels (internal; the public ABI is pa.h).
// Each launcher assumes its arguments were validated by pa_api.cpp and only
// enqueues work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;   // tokens per KV block
constexpr int kHeadDim = 128;    // elements per head row
constexpr int kDecodeRows = 8;   // most query rows per (sequence, KV head) the decode kernel takes

hipError_t launch_kv_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, hipStream_t stream);

// Split-K decode over sequences with n_s * G <= 8 query rows per KV head.
// The workspace holds per-(sequence, KV head) completion counters, which must
// be zero before the first call and are left zero by every call, followed by
// the partitions' (m, l, acc) records.
struct DecodePlan {
  int32_t rows;            // query rows per (sequence, KV head) the kernel instance holds (1,2,4,8)
  int32_t part_blocks;     // KV blocks per partition
  int32_t max_parts;       // partitions of the longest sequence
};
DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t max_context_len, int32_t max_query_len);
size_t decode_workspace_bytes(const DecodePlan& plan, int32_t num_seqs, int32_t num_kv_heads);

hipError_t launch_decode(bool is_bf16, const DecodePlan& plan, void* out, const void* q,
                         const void* k_pool, const void* v_pool, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, float scale, void* workspace,
                         hipStream_t stream);

// Matrix-core prefill over sequences with n_s * G > 8 query rows per KV head.
hipError_t launch_prefill(bool is_bf16, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                          float scale, hipStream_t stream);

}  // namespace pa

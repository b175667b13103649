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
constexpr int kRecFloats = 132;  // partial (m, l, acc) record: acc[128], m, l, 2 pad (16-B aligned)
constexpr int kWgRows = 128;     // query rows per narrow prefill workgroup
constexpr int kWideWgRows = 256; // query rows per wide prefill workgroup (4 x 64 or 8 x 32)
// Calls that may prefill with at most this many sequences have the decode
// kernel rank the prefill's work (one sequence per lane of one wave) instead
// of a launch of the ranking kernel.
constexpr int kRankInDecodeSeqs = 64;

// Shared-prefix cascade for decode.  Consecutive one-token sequences whose
// block tables start with the same physical blocks (prefix sharing through
// identical table entries) form a group of at most kCascadeMaxMembers; the
// group's common full blocks (at least kCascadeMinBlocks, never the block
// holding a member's last key) are attended once for all members' rows and
// split over at most kPrefixChunks workgroups per KV head (chunks of at
// least kChunkTiles 64-key tiles), each leaving one (m, l, acc) record per
// row that the decode kernel merges with its own.
constexpr int kCascadeMinBlocks = 4;
constexpr int kCascadeMaxMembers = 32;
constexpr int kPrefixChunks = 8;
constexpr int kChunkTiles = 16;  // 64-key tiles per prefix chunk, at least (if there are)

// Block dst_ids[i] of (dst_k, dst_v) becomes a copy of block src_ids[i] of
// (src_k, src_v) (device id arrays; the pools may be the same, or one of them
// pinned host memory at its device address).  A null id array stands for
// 0, 1, ..., num_copies - 1.
hipError_t launch_copy_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* src_ids, const int32_t* dst_ids, int32_t num_copies,
                              int32_t src_blocks, int32_t dst_blocks, int32_t num_kv_heads,
                              hipStream_t stream);

// Quantized pages (qpage.h): page page_ids[i] of qpool becomes the
// quantized form of the 128 tokens held by blocks src_blocks[i][0..7].
hipError_t launch_quantize_pages(bool is_bf16, void* qpool, const void* k_pool,
                                 const void* v_pool, const int32_t* page_ids,
                                 const int32_t* src_blocks, int32_t num_encode,
                                 int32_t num_pages, int32_t num_blocks, int32_t num_kv_heads,
                                 hipStream_t stream);

hipError_t launch_kv_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, hipStream_t stream);

// Decode of sequences with n_s * G <= 8 query rows per KV head.  Its work,
// Hkv * (blocks to decode) units per sequence, is cut into equal slices, one
// per wave of a grid that is resident at once.  The workspace holds
// per-(sequence, KV head) completion counters, which must be zero before the
// first call and are left zero by every call, and the records of pairs that
// a slice edge cuts.
constexpr int kMinChunk = 4;  // least units (KV head x block) per wave
struct DecodePlan {
  int32_t rows;   // query rows per (sequence, KV head) the kernel instance holds (1,2,4,8); 0: no decode
  int32_t waves;  // grid size
};
DecodePlan plan_decode(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t max_context_len, int32_t max_query_len);

// Byte offsets of the workspace regions (each 256-B aligned).  First the
// zero region, bytes that must be zero when a call starts and that every
// completed call leaves at zero, at offsets that do not depend on the call:
//   item_count int32 at 0        cascade: work items planned (reset by the decode)
//   counters   [S][Hkv] uint32 at 256  decode: slices of a cut pair finished
// then, rewritten by every call before they are read:
//   starts     [S][2] int32      cascade: first block left to decode, prefix chunks
//   items      [max_items][8] int32  cascade: (group, chunk, KV head) work items
//   prefix     [S][Hkv][G][kPrefixChunks][kRecFloats] float  cascade records
//   records    [waves][2][rows][kRecFloats] float  decode: records of cut pairs
//   queue      [8] int32         prefill: next item of each XCD's queue
//   order      [S] int32         prefill: sequences by decreasing prefill work
// min_zero_bytes reserves a zero region of at least that size (a workspace
// shared by calls of different sizes).
struct WorkspaceLayout {
  bool cascade;
  bool prefill;
  int32_t max_items;
  size_t zero_bytes;
  size_t item_count, counters, starts, items, prefix, records, queue, order, total;
};
constexpr int kOrderMaxSeqs = 1024;  // one workgroup ranks them, one sequence per thread
WorkspaceLayout workspace_layout(const DecodePlan& plan, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t max_context_len,
                                 int32_t max_query_len, size_t min_zero_bytes = 0,
                                 bool allow_cascade = true);

hipError_t launch_decode(bool is_bf16, const DecodePlan& plan, const WorkspaceLayout& ws,
                         void* out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, const int32_t* query_start_loc,
                         int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         float scale, void* workspace, hipStream_t stream,
                         bool rank_prefill = false);

// Decode over sequences whose first quant_lens[s] keys (a multiple of 128)
// are quantized pages of qpool reached through page_tables, the rest 16-bit
// blocks of the pools; the layout must come with allow_cascade false.
struct QuantArgs {
  const uint8_t* qpool;
  const int32_t* page_tables;
  int32_t max_pages;
  const int32_t* quant_lens;
};
hipError_t launch_decode_quant(bool is_bf16, const DecodePlan& plan, const WorkspaceLayout& ws,
                               void* out, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               float scale, const QuantArgs& qa, void* workspace,
                               hipStream_t stream);

// Shared-prefix pass (only when ws.cascade), two launches: the plan (every
// sequence's starts entry and the work items) and the prefix attention (the
// records of grouped sequences).  Runs before the decode.
hipError_t launch_cascade(bool is_bf16, const WorkspaceLayout& ws, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                          float scale, void* workspace, hipStream_t stream);

// Matrix-core prefill over sequences with n_s * G > 8 query rows per KV head.
// A one-workgroup pass first ranks the sequences by prefill work so that the
// longest start first, and empties the XCD work queues of the persistent
// prefill kernel.
hipError_t launch_prefill(bool is_bf16, const WorkspaceLayout& ws, void* out, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start_loc, int32_t num_seqs,
                          int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                          float scale, void* workspace, hipStream_t stream,
                          bool ranked = false);

}  // namespace pa

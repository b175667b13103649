/*
 * pa.h -- C ABI of the generalized paged-attention library (libpa.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes
 * -------------------------
 * K and V of one attention layer live in a pool of fixed 16-token blocks
 * (SOSP 2023 PagedAttention explainer, "PagedAttentionアルゴリズム": blocks of
 * B = 16 tokens).  Each sequence reaches its blocks through a row of a block
 * table mapping logical block j to a physical block (same page, "ブロック
 * テーブルによるメモリ管理").  Sequences may share physical blocks by holding
 * identical table entries (same page, "Copy-on-Writeによるメモリ共有" and
 * "Prefix Caching").
 *
 * A batch mixes decode sequences (one new query token) and prefill sequences
 * (a run of new tokens that are causal among themselves and see the whole
 * cached history), with ragged query lengths, non-contiguous KV and a causal
 * mask applied inside the kernel (Stateful LLM Serving with Pensieve
 * explainer, "汎化PagedAttentionカーネル").  Each output row is
 * softmax(q K^T * scale) V over the keys that row may see (PagedAttention
 * explainer, "PagedAttentionアルゴリズム", the attention equation).
 *
 * Layouts (all row-major, all device memory owned by the caller)
 * --------------------------------------------------------------
 *   q, out        [total_q, num_q_heads, head_dim]         fp16 or bf16
 *   k_new, v_new  [num_tokens, num_kv_heads, head_dim]     fp16 or bf16
 *   k_pool,v_pool [num_blocks, num_kv_heads, block_size, head_dim]
 *                 one (block, kv head) tile is block_size*head_dim contiguous
 *                 elements (4 KiB for 16 x 128 x 2 B).  One pool per layer.
 *   slot_mapping  [num_tokens] int32: slot = block * block_size + offset,
 *                 -1 = do not write this token.
 *   block_tables  [num_seqs, max_blocks_per_seq] int32 physical block ids.
 *   context_lens  [num_seqs] int32: C_s, every key sequence s can see,
 *                 including its n_s new tokens (written by pa_kv_write first).
 *   query_start_loc [num_seqs + 1] int32: query rows of sequence s are
 *                 query_start_loc[s] .. query_start_loc[s+1]-1;
 *                 query_start_loc[0] = 0, query_start_loc[num_seqs] = total_q.
 *
 * With n_s = query_start_loc[s+1] - query_start_loc[s], query row i of
 * sequence s (0 <= i < n_s) is position C_s - n_s + i and sees keys
 * 0 .. C_s - n_s + i (bottom-right causal).  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads) (grouped-query attention).
 *
 * Supported: block_size == 16, head_dim == 128, dtype PA_F16 or PA_BF16,
 * num_q_heads a multiple of num_kv_heads.  Arithmetic: products and sums in
 * fp32, output rounded to the input dtype (round to nearest even).
 *
 * Ownership, streams, errors
 * --------------------------
 * Every pointer is device memory owned by the caller.  The library never
 * allocates, frees or synchronises; it keeps no state between calls and is
 * safe to call from several threads.  Work is enqueued on `stream` (a
 * hipStream_t; NULL is the legacy default stream) and runs asynchronously.
 * Only host-visible arguments are validated, always before anything is
 * enqueued; on error nothing is launched.  Device-resident metadata is a
 * precondition the kernels do not check (pa_check_batch below checks it on
 * host copies):
 *   - block_tables[s][j] in [0, num_blocks) for j < ceil(C_s / 16)
 *     (entries past that are never read and may hold anything);
 *   - 0 <= n_s <= C_s <= max_context_len, n_s <= max_query_len;
 *   - slots distinct and in [0, num_blocks * 16), or -1;
 *   - no slot lies in a block another sequence also references (copy the
 *     block first: PagedAttention explainer, "Copy-on-Writeによるメモリ共有").
 * Slots at positions >= C_s of a sequence's last block may hold any bits,
 * NaN included; they never reach the output.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k/v, pools and out. */
typedef enum { PA_F16 = 0, PA_BF16 = 1 } pa_dtype;

/* Return codes. */
typedef enum {
  PA_OK = 0,
  PA_EINVAL = 1,        /* null pointer, negative size, inconsistent sizes */
  PA_EUNSUPPORTED = 2,  /* block_size != 16, head_dim != 128, unknown dtype */
  PA_EWORKSPACE = 3,    /* workspace missing or smaller than required */
  PA_EHIP = 4,          /* the HIP runtime reported a launch error */
  PA_ESCRATCH = 5,      /* pa_attention_noalloc: the call needs more than the
                           library's static scratch array holds */
  PA_ENOBLOCKS = 6      /* pa_bm_append (pa_blocks.h): too few free blocks */
} pa_status;

/* Version of this ABI (bumped on any signature or semantics change). */
int32_t pa_abi_version(void);

/* Static, human-readable name of a pa_status value (never NULL).  Takes and
 * the entry points return int32_t rather than pa_status, so that the ABI's
 * integer width does not depend on the compiler's choice of enum size. */
const char* pa_status_str(int32_t status);

/*
 * pa_kv_write -- scatter new K/V rows into their pool slots.
 *
 * For every token t with slot_mapping[t] >= 0 and every KV head h:
 *   k_pool[slot / 16][h][slot % 16][:] = k_new[t][h][:]   (same for V)
 * A new token is appended into its sequence's current block, or the block the
 * caller allocated for it (PagedAttention explainer, "ブロックテーブルによる
 * メモリ管理").  The copy is bit-exact.  num_tokens == 0 is a no-op.
 * Errors: PA_EINVAL for a null pointer (when num_tokens > 0) or negative
 * sizes; PA_EUNSUPPORTED for block_size != 16, head_dim != 128 or an unknown
 * dtype; PA_EHIP if the launch fails.
 */
int32_t pa_kv_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                    const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t dtype, void* stream);

/*
 * pa_attention_workspace_size -- bytes of device workspace pa_attention needs
 * for these sizes (0 is possible).  num_kv_heads sizes the per-(sequence, KV
 * head) counters below.  The decode splits the batch's work into equal
 * slices, one per wave; when there is more than one wave the workspace
 * holds, per (sequence, KV head), a counter of the finished slices that cut
 * it, and per wave the (max, sum, unnormalised output) records of the two
 * pairs its slice may cut, until the last slice of a pair merges them.  For
 * batches that may share prefix blocks it also holds each sequence's
 * shared-prefix plan, its work-item count and the (max, sum, output) records
 * of the shared prefixes; and, for batches that may prefill, the prefill's
 * work queues and its order of the sequences by decreasing prefill work.
 *
 * Zero region.  The item count (bytes 0..3) and the counters (from byte 256,
 * 4 * num_seqs * num_kv_heads bytes; present in every call that needs a
 * workspace, whatever else it holds) must be zero when a call starts, and
 * every completed call leaves them at zero; everything after them is
 * rewritten by each call before it is read.  So: zero-fill a new workspace
 * once before its first use; it can then be reused without clearing by any
 * later call whose num_seqs * num_kv_heads is at most that of every call it
 * served since it was zero-filled (a call with more pairs needs a fresh
 * zero-fill: bytes past the earlier calls' counters hold their other data).
 * Calls that share a workspace must be ordered (same stream): overlapping
 * calls on one workspace race.  Returns 0 for invalid sizes.
 */
size_t pa_attention_workspace_size(int32_t num_seqs, int32_t total_q, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t max_query_len);

/*
 * pa_attention -- generalized paged attention over one layer.
 *
 * out[t][h][:] = sum_j softmax_j(scale * <q[t][h], K_j>) V_j over the keys
 * row t may see (see the header comment).  Sequences with n_s * G <= 8 query
 * rows per KV head (G = num_q_heads / num_kv_heads) run on a split-K decode
 * kernel that gives every wave an equal share of the batch's K/V blocks; the
 * pieces of a (sequence, KV head) cut between waves are merged with the
 * rescaling of an online softmax (KV-cache textbook ch.6, FlashAttention-2
 * logsumexp).  The others run on a matrix-core prefill kernel.  A sequence with n_s == 0 writes no rows.
 * Consecutive one-token sequences whose block tables start with the same
 * physical blocks (prefix sharing through identical table entries,
 * PagedAttention explainer, "メモリ共有") are found on the device: their
 * common full blocks are attended once for the whole group on the matrix
 * cores, and each member's decode covers only its own tail and merges.
 *
 * max_query_len and max_context_len are host-side upper bounds of n_s and C_s;
 * they size the launch, so no device memory is read on the host.
 * workspace must be at least pa_attention_workspace_size(...) bytes (NULL if
 * that is 0) and zero-filled before its first use (see above).
 * scale must be finite and positive (the pages' 1/sqrt(head_dim) is).
 * Errors: PA_EINVAL (null pointer, negative size, num_q_heads not a multiple
 * of num_kv_heads, max_blocks_per_seq too small for max_context_len, scale
 * not finite and positive, or a batch with decode rows whose
 * num_seqs * num_kv_heads * ceil(max_context_len / 16) reaches 2^32),
 * PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP, all before anything is enqueued
 * except PA_EHIP.
 */
int32_t pa_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start_loc,
                     int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                     int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                     int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_attention_noalloc -- pa_attention without a caller workspace, for
 * callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, results and
 * errors as pa_attention, minus workspace and workspace_bytes.  The
 * workspace is a static device array of the library (64 MiB, one copy per
 * GPU, held until the process ends); nothing is allocated.  Its first 256 KiB
 * are the zero region of every call (see pa_attention_workspace_size), which
 * limits a call to 65,472 (sequence, KV head) pairs; a call with more, or
 * whose other regions need more than the rest of the array (their size is
 * pa_attention_workspace_size minus its zero region), returns PA_ESCRATCH
 * before anything is enqueued.  The first call on a GPU also enqueues one
 * kernel that clears the zero region.  Every call on a GPU shares that GPU's
 * array: calls that overlap on one GPU (other streams, other threads) race;
 * order them.  out, q, pools and metadata are the caller's, as for
 * pa_attention.
 */
int32_t pa_attention_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* query_start_loc,
                             int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                             int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             float scale, int32_t dtype, void* stream);

/*
 * pa_check_batch: the device-resident preconditions listed at the top of this
 * header, checked on HOST copies of the metadata (every pointer here is host
 * memory, read only).  The kernels take tables, lengths and slots on trust; a
 * caller whose bookkeeping is in doubt runs the batch through this first and
 * gets PA_EINVAL with the first bad entry named in msg, instead of a read or
 * write outside the pool on the GPU.  No HIP call is made.
 *
 * Checked, in this order:
 *   - query_start_loc[0] == 0, non-decreasing, query_start_loc[num_seqs] ==
 *     total_q (the ragged rows of the Pensieve explainer's
 *     "汎化PagedAttentionカーネル");
 *   - 0 <= n_s <= C_s <= max_context_len and n_s <= max_query_len;
 *   - ceil(C_s / 16) <= max_blocks_per_seq and block_tables[s][j] in
 *     [0, num_blocks) for j < ceil(C_s / 16) (PagedAttention explainer,
 *     "ブロックテーブルによるメモリ管理");
 *   - each of the num_slots slots is -1 or in [0, num_blocks * 16), no slot
 *     appears twice, and no slot lies in a block that two or more table
 *     entries of this batch name (a write into a shared block needs its copy
 *     first: same explainer, "Copy-on-Writeによるメモリ共有").  References are
 *     counted over this batch's tables only;
 *   - if slots_are_new_tokens != 0: num_slots == total_q and the slot of row
 *     i of sequence s is -1 or the table position of C_s - n_s + i (the
 *     kv_write of a step writes exactly the keys its query rows add).
 * slot_mapping may be NULL when num_slots == 0.  msg receives a
 * NUL-terminated message (truncated to msg_bytes - 1 characters; "" on
 * success); msg may be NULL when msg_bytes == 0.  Returns PA_OK or PA_EINVAL.
 */
int32_t pa_check_batch(const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* context_lens, const int32_t* query_start_loc,
                       int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                       int32_t max_context_len, int32_t num_blocks, const int32_t* slot_mapping,
                       int32_t num_slots, int32_t slots_are_new_tokens, char* msg,
                       size_t msg_bytes);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */

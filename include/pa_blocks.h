/*
 * pa_blocks.h -- paged KV block management for libpa (host side) and the
 * device copy that copy-on-write needs.
 *
 * A pool holds num_blocks physical blocks of 16 tokens (SOSP 2023
 * PagedAttention explainer, "PagedAttentionアルゴリズム": B = 16).  Each
 * sequence owns a block table mapping its logical blocks to physical ones
 * (same page, "ブロックテーブルによるメモリ管理").  A new token goes into the
 * sequence's current block while it has room, and into a block taken from
 * the free list once it is full; a finished sequence returns its blocks to
 * the free list at once, so a sequence of C tokens holds ceil(C / 16) blocks
 * and wastes at most 15 slots (same section).  Sequences share a physical
 * block by holding the same table entry: the samples of one prompt
 * (pa_bm_fork) and a request that reuses an earlier request's prefix
 * (pa_bm_share_prefix) ("Copy-on-Writeによるメモリ共有", "Prefix Caching").
 * Every block has a reference count; a write into a block whose count is 2
 * or more first copies the block (copy-on-write, same section).  Appends only
 * ever write at a sequence's end, so the one block a write can hit is the
 * sequence's partly filled last block.
 *
 * The manager lives in host memory and touches no device memory: pa_bm_append
 * hands back the slots of the new tokens (for pa_kv_write) and the block
 * copies that must run first (for pa_copy_blocks); pa_bm_tables writes block
 * tables and context lengths in the layout pa_attention reads.  Policies the
 * pages leave open: the free list is a queue (blocks are taken from its front,
 * returned to its back, a sequence's blocks in table order) with an initial
 * order the caller may give; a copy-on-write takes its block before the
 * append's new blocks; sequence ids count up from 0 and are never reused.
 *
 * Threads: each manager call takes the manager's own lock, so calls on one
 * manager from several threads are safe (and serialised).
 * Errors: PA_EINVAL (null pointer, unknown or freed sequence, bad size),
 * PA_ENOBLOCKS (the free list cannot hold the append; nothing changes).
 */
#ifndef PA_BLOCKS_H
#define PA_BLOCKS_H

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager of num_blocks blocks, all free.  free_order (host memory, may be
 * NULL for 0, 1, ..., num_blocks - 1) lists every block id once: the free
 * list's initial order.  *out receives the manager (destroy it with
 * pa_bm_destroy).  PA_EINVAL if num_blocks <= 0 or free_order is not a
 * permutation of 0 .. num_blocks - 1. */
int32_t pa_bm_create(int32_t num_blocks, const int32_t* free_order, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new empty sequence; *seq receives its id. */
int32_t pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq);

/* A new sequence holding parent's tokens in parent's blocks (every one of
 * them gains a reference): a sample of the same prompt. */
int32_t pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child);

/* A new sequence holding the first num_tokens tokens of src, in src's first
 * ceil(num_tokens / 16) blocks (each gains a reference): prefix caching by
 * sharing table entries.  0 <= num_tokens <= src's length. */
int32_t pa_bm_share_prefix(pa_block_manager* bm, int32_t src, int32_t num_tokens,
                           int32_t* seq);

/* Blocks an append of num_tokens to seq would take from the free list
 * (copy-on-write included), or -1 for an invalid call. */
int32_t pa_bm_blocks_needed(const pa_block_manager* bm, int32_t seq, int32_t num_tokens);

/* Room for num_tokens new tokens at seq's end.  slots (host, num_tokens
 * entries) receives each new token's slot, physical block * 16 + offset, in
 * order.  copy_src / copy_dst (host, one entry each) receive the block copy
 * that must run before the new tokens are written (pa_copy_blocks), and
 * *num_copies their count, 0 or 1: a copy happens when seq's last block is
 * partly filled and shared.  PA_ENOBLOCKS, changing nothing, if the free
 * list is too short.  Run each append's copy, then its writes, in the order
 * of the appends (a later append may write into a block an earlier copy
 * reads); copies of appends with no fork or share between them may be
 * batched ahead of those appends' writes. */
int32_t pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* slots,
                     int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies);

/* seq is finished: each of its blocks loses a reference, and a block that
 * no sequence references goes back to the free list.  The id stays invalid. */
int32_t pa_bm_free_sequence(pa_block_manager* bm, int32_t seq);

/* Free blocks, a block's reference count, a sequence's length in tokens;
 * -1 for an invalid argument. */
int32_t pa_bm_num_free(const pa_block_manager* bm);
int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block);
int32_t pa_bm_length(const pa_block_manager* bm, int32_t seq);

/* Block tables and context lengths of num_seqs sequences, in pa_attention's
 * layout: block_tables (host) [num_seqs][max_blocks_per_seq] int32, entries
 * past a sequence's blocks set to -1; context_lens (host) [num_seqs].
 * PA_EINVAL if a sequence is invalid or holds more than max_blocks_per_seq
 * blocks. */
int32_t pa_bm_tables(const pa_block_manager* bm, const int32_t* seqs, int32_t num_seqs,
                     int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens);

/*
 * pa_copy_blocks -- block dst[i] of both pools becomes a copy of block src[i]
 * (all KV heads, all 16 slots, K and V), bit for bit: the copy of
 * copy-on-write (PagedAttention explainer, "Copy-on-Writeによるメモリ共有").
 * k_pool, v_pool: [num_blocks, num_kv_heads, block_size, head_dim], device.
 * src, dst: device int32 arrays of num_copies block ids.  Preconditions
 * (device memory, not checked on the host): the dst ids are distinct and
 * none is a src id.  An id outside [0, num_blocks) makes its copy a no-op.
 * num_copies == 0 is a no-op.  Enqueued on stream; run it before the
 * pa_kv_write of the tokens whose append asked for it.
 * Errors: PA_EINVAL (null pointer with num_copies > 0, negative sizes),
 * PA_EUNSUPPORTED (block_size != 16, head_dim != 128, unknown dtype), PA_EHIP.
 */
int32_t pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* src, const int32_t* dst,
                       int32_t num_copies, int32_t num_blocks, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_swap_blocks -- block dst_ids[i] of the destination pools becomes a copy
 * of block src_ids[i] of the source pools (all KV heads, all 16 slots, K and
 * V), bit for bit: swap-out (GPU pool -> CPU tier) and swap-in (CPU tier ->
 * GPU pool) of a two-tier KV cache (Pensieve explainer, "GPU-CPU 2層キャッシュ
 * 構造").  Swap-in runs per layer, so that layer i+1's transfer on one
 * stream overlaps layer i's attention on another ("パイプライン化された
 * swap-in").  One launch moves the whole list: every (block, head) tile is
 * read where it lies and written where it goes, so scattered 16-token blocks
 * need neither a staging buffer nor one call per block (KV-cache textbook
 * ch.14: 16-token pages are too small a transfer unit on their own).
 * Pools: [src|dst]_num_blocks x [num_kv_heads, block_size, head_dim], each
 * either device memory or pinned host memory (hipHostMalloc, or a torch
 * tensor made with pin_memory=True), which the GPU reads and writes across
 * the host link; pageable host memory is refused (PA_EINVAL).  src_ids and
 * dst_ids: device int32 arrays of num_copies ids; the dst ids are distinct,
 * and when source and destination are the same pools, none is a src id.  An
 * id outside its pool makes its copy a no-op.  Ownership: all the caller's;
 * the library allocates nothing.  Enqueued on stream.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED, PA_EHIP, before anything is enqueued
 * except PA_EHIP.
 *
 * Measured on MI355X: this kernel reaches the host link's rate (57 GB/s,
 * that of a plain copy-engine transfer), but while it reads host memory,
 * kernels on other streams slow severalfold (a decode layer 58 -> 150 us).
 * Swap-in beside attention therefore goes through pa_swap_in_staged, which
 * leaves the host link to the copy engines.
 */
int32_t pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                       const int32_t* src_ids, const int32_t* dst_ids, int32_t num_copies,
                       int32_t src_num_blocks, int32_t dst_num_blocks, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_swap_in_staged -- swap-in of one layer's evicted blocks, the way that
 * overlaps attention (Pensieve explainer, "パイプライン化されたswap-in";
 * KV-cache textbook ch.14: move a contiguous run across the link, scatter
 * the 16-token blocks on arrival).  The CPU tier keeps the layer's evicted
 * blocks as one contiguous run, host_k / host_v [num_copies, num_kv_heads,
 * block_size, head_dim] in pinned host memory.  The copy engines move the
 * run into staging_k / staging_v (device, at least as large), then a kernel
 * scatters staged block i into block dst_ids[i] of k_pool / v_pool
 * ([num_blocks, ...], device); dst_ids: device int32 [num_copies], distinct.
 * All enqueued on stream, in that order.  The staging run is the caller's
 * and must not be reused before the scatter has run.
 * Errors: PA_EINVAL (null pointer, negative size, a host run that is not
 * pinned host memory, a staging run or pool that is not device memory),
 * PA_EUNSUPPORTED, PA_EHIP.
 */
int32_t pa_swap_in_staged(void* k_pool, void* v_pool, const void* host_k, const void* host_v,
                          void* staging_k, void* staging_v, const int32_t* dst_ids,
                          int32_t num_copies, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_swap_out_staged -- the reverse: blocks src_ids[i] of k_pool / v_pool are
 * gathered into staging block i on the device, then the copy engines move
 * the run to host_k / host_v (pinned host memory, [num_copies, ...]).  Same
 * arguments and errors as pa_swap_in_staged.  The host run holds the data
 * once the stream has passed the call.
 */
int32_t pa_swap_out_staged(void* host_k, void* host_v, const void* k_pool, const void* v_pool,
                           void* staging_k, void* staging_v, const int32_t* src_ids,
                           int32_t num_copies, int32_t num_blocks, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCKS_H */

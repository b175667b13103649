/*
 * pa_quant.h -- quantized KV pages for libpa: 2-bit keys and values with the
 * key channels of largest magnitude promoted to 4 bits, and decode attention
 * that reads them (KV-cache textbook ch.22, the Kitty passage).
 *
 * Format.  A quantized page holds 128 tokens of one KV head: a quantization
 * group of 128 tokens is one page, which keeps quantized pages compatible
 * with paged attention, and a page is quantized once, when its 128 tokens
 * are complete (the heavy work amortised over 128 decode steps).  Keys are
 * quantized per channel along the page's tokens, values per token along its
 * channels; every group is asymmetric and uniform: mn = min x, step =
 * (max x - mn) / levels, code = min(levels, rint((x - mn) / step)), all in
 * float32 with round-to-nearest-even (code 0 when step is 0), standing for
 * mn + code * step.  levels = 3 (2 bits), except for the 16 key channels of
 * largest float32 sum of |k| over the page's tokens (ties to the lower
 * channel), which get levels = 15 (4 bits, the lower end of the passage's
 * 12.5-25%).  A promoted channel's code is split: its low 2 bits sit in the
 * dense plane every channel has, its high 2 bits in a small sparse plane of
 * the promoted channels only, so every channel is read the same way.  The
 * passage leaves the value side open; values are read here as the KIVI
 * arrangement the same chapter names (per token, 2 bits).
 * A pool of quantized pages is [num_pages][num_kv_heads][PA_QPAGE_BYTES]
 * bytes in device memory; the byte layout inside a page is the library's
 * (it follows the decode's lane order) and opaque to callers.
 * One page for one KV head: 10,816 bytes, against 65,536 for the same 128
 * tokens of K and V in fp16/bf16 (6.06x smaller).
 *
 * Ownership and streams as in pa.h: caller's device memory, work enqueued
 * on stream, nothing allocated or synchronised.
 */
#ifndef PA_QUANT_H
#define PA_QUANT_H

#include <stdint.h>

#include "pa.h"

#define PA_QPAGE_TOKENS 128
#define PA_QPAGE_BYTES 10816

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pa_quantize_pages -- page page_ids[i] of qpool becomes the quantized form
 * of the 128 tokens that blocks src_blocks[i][0..7] of k_pool / v_pool hold,
 * in that order, every KV head.  page_ids: device int32 [num_encode],
 * distinct; src_blocks: device int32 [num_encode][8].  k_pool / v_pool:
 * [num_blocks, num_kv_heads, block_size, head_dim], fp16 or bf16.  A page or
 * block id out of range makes its page a no-op.  The blocks may be freed
 * (their ids reused) once the stream has passed the call.
 * Errors: PA_EINVAL, PA_EUNSUPPORTED (block_size != 16, head_dim != 128,
 * unknown dtype), PA_EHIP.
 */
int32_t pa_quantize_pages(void* qpool, const void* k_pool, const void* v_pool,
                          const int32_t* page_ids, const int32_t* src_blocks, int32_t num_encode,
                          int32_t num_pages, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t dtype, void* stream);

/*
 * pa_attention_quant -- decode attention (pa.h's pa_attention) over
 * sequences whose first quant_lens[s] keys, a multiple of 128, are quantized
 * pages page_tables[s][0 .. quant_lens[s]/128 - 1] of qpool, and whose other
 * keys are 16-bit blocks of k_pool / v_pool reached through block_tables
 * from block quant_lens[s] / 16 on (the entries before it are never read).
 * Every query row sees every quantized key: quant_lens[s] <= context_lens[s]
 * - n_s (device precondition).  Decode only: max_query_len * (num_q_heads /
 * num_kv_heads) <= 8, else PA_EUNSUPPORTED.  The workspace is sized by
 * pa_attention_workspace_size with the same bounds and follows its rules.
 * Shared prefixes are not attended once per group here (every sequence
 * reads its own pages).  Other arguments, results and errors as
 * pa_attention; PA_EINVAL also for a null page table or quant_lens.
 */
int32_t pa_attention_quant(void* out, const void* q, const void* qpool,
                           const int32_t* page_tables, int32_t max_pages_per_seq,
                           const int32_t* quant_lens, int32_t num_pages, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q,
                           int32_t max_query_len, int32_t max_context_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, float scale, int32_t dtype, void* workspace,
                           size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_QUANT_H */

// pa_check_batch (include/pa.h): the device-resident preconditions of
// pa_kv_write and pa_attention, checked on host copies of the metadata.
//
// The kernels take block tables, lengths, query offsets and slots on trust
// (reading them back to the host on every call would cost a synchronisation).
// A caller whose bookkeeping is in doubt -- the tests and the benchmark do
// this before every GPU call -- runs the same batch through this check first
// and gets an error naming the first bad entry instead of an access outside
// the pool.  Pure host code: no HIP call, no allocation beyond one sort buffer
// and one count per block.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <vector>

#include "pa.h"

namespace {

constexpr int64_t kBlock = 16;

int32_t fail(char* msg, size_t msg_bytes, const char* fmt, ...) {
  if (msg && msg_bytes > 0) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, msg_bytes, fmt, ap);
    va_end(ap);
  }
  return PA_EINVAL;
}

}  // namespace

extern "C" int32_t pa_check_batch(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, const int32_t* query_start_loc,
                                  int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                                  int32_t max_context_len, int32_t num_blocks,
                                  const int32_t* slot_mapping, int32_t num_slots,
                                  int32_t slots_are_new_tokens, char* msg, size_t msg_bytes) {
  if (msg && msg_bytes > 0) msg[0] = '\0';
  if (num_seqs < 0 || total_q < 0 || max_query_len < 0 || max_context_len < 0 ||
      num_blocks < 0 || max_blocks_per_seq < 0 || num_slots < 0)
    return fail(msg, msg_bytes, "negative size");
  if (num_seqs > 0 && (!context_lens || !query_start_loc))
    return fail(msg, msg_bytes, "context_lens or query_start_loc is NULL");
  if (num_slots > 0 && !slot_mapping) return fail(msg, msg_bytes, "slot_mapping is NULL");
  if ((int64_t)num_blocks * kBlock > INT32_MAX)
    return fail(msg, msg_bytes, "num_blocks * 16 exceeds the int32 slot range");

  // Query offsets: start at 0, never decrease, end at total_q.
  if (num_seqs > 0) {
    if (query_start_loc[0] != 0)
      return fail(msg, msg_bytes, "query_start_loc[0] = %d, not 0", query_start_loc[0]);
    if (query_start_loc[num_seqs] != total_q)
      return fail(msg, msg_bytes, "query_start_loc[%d] = %d, not total_q = %d", num_seqs,
                  query_start_loc[num_seqs], total_q);
  } else if (total_q != 0) {
    return fail(msg, msg_bytes, "total_q = %d with no sequences", total_q);
  }

  // Lengths, and every block a sequence reads.  References are counted over
  // this batch's tables: the blocks a write must not touch are those more
  // than one table entry names.
  std::vector<int32_t> refs((size_t)num_blocks, 0);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t lo = query_start_loc[s], hi = query_start_loc[s + 1];
    if (hi < lo)
      return fail(msg, msg_bytes, "query_start_loc decreases at sequence %d (%d -> %d)", s, lo,
                  hi);
    const int64_t n = (int64_t)hi - lo, C = context_lens[s];
    if (C < 0 || C > max_context_len)
      return fail(msg, msg_bytes, "sequence %d: context length %lld outside [0, %d]", s,
                  (long long)C, max_context_len);
    if (n > C)
      return fail(msg, msg_bytes, "sequence %d: %lld new tokens but context length %lld", s,
                  (long long)n, (long long)C);
    if (n > max_query_len)
      return fail(msg, msg_bytes, "sequence %d: %lld new tokens exceed max_query_len %d", s,
                  (long long)n, max_query_len);
    const int64_t nb = (C + kBlock - 1) / kBlock;
    if (nb > max_blocks_per_seq)
      return fail(msg, msg_bytes, "sequence %d: %lld blocks exceed max_blocks_per_seq %d", s,
                  (long long)nb, max_blocks_per_seq);
    if (nb > 0 && !block_tables) return fail(msg, msg_bytes, "block_tables is NULL");
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks)
        return fail(msg, msg_bytes, "sequence %d: block_tables[%d][%lld] = %d outside [0, %d)",
                    s, s, (long long)j, b, num_blocks);
      ++refs[(size_t)b];
    }
  }

  // Slots: each in range or -1, no two alike, none in a shared block.
  std::vector<int32_t> sorted;
  sorted.reserve((size_t)num_slots);
  for (int32_t t = 0; t < num_slots; ++t) {
    const int32_t slot = slot_mapping[t];
    if (slot == -1) continue;
    if (slot < 0 || (int64_t)slot >= (int64_t)num_blocks * kBlock)
      return fail(msg, msg_bytes, "slot_mapping[%d] = %d outside [0, %lld) and not -1", t, slot,
                  (long long)num_blocks * kBlock);
    if (refs[(size_t)(slot / kBlock)] >= 2)
      return fail(msg, msg_bytes,
                  "slot_mapping[%d] = %d writes into block %d, which %d table entries "
                  "share (copy it first)",
                  t, slot, slot / (int32_t)kBlock, refs[(size_t)(slot / kBlock)]);
    sorted.push_back(slot);
  }
  std::sort(sorted.begin(), sorted.end());
  const auto dup = std::adjacent_find(sorted.begin(), sorted.end());
  if (dup != sorted.end()) return fail(msg, msg_bytes, "slot %d is written twice", *dup);

  // Optionally: token t of the batch is query row t, and its slot is the
  // position that row stands for, C_s - n_s + i, through the sequence's table.
  if (slots_are_new_tokens) {
    if (num_slots != total_q)
      return fail(msg, msg_bytes, "%d slots for %d new tokens", num_slots, total_q);
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t lo = query_start_loc[s], n = query_start_loc[s + 1] - lo;
      const int64_t C = context_lens[s];
      for (int32_t i = 0; i < n; ++i) {
        const int32_t slot = slot_mapping[lo + i];
        if (slot == -1) continue;
        const int64_t pos = C - n + i;
        const int64_t want =
            (int64_t)block_tables[(int64_t)s * max_blocks_per_seq + pos / kBlock] * kBlock +
            pos % kBlock;
        if (slot != want)
          return fail(msg, msg_bytes,
                      "sequence %d row %d (position %lld): slot %d, but its table puts it at %lld",
                      s, i, (long long)pos, slot, (long long)want);
      }
    }
  }
  return PA_OK;
}

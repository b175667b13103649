// Host-side paged KV block manager of libpa (declared in include/pa_blocks.h):
// a free-list queue of physical blocks, a reference count per block and a
// block table per sequence (SOSP 2023 PagedAttention explainer,
// "ブロックテーブルによるメモリ管理", "Copy-on-Writeによるメモリ共有",
// "Prefix Caching").  Plain host code: it never touches device memory.
#include <stdint.h>

#include <mutex>
#include <vector>

#include "pa_blocks.h"

namespace {
constexpr int32_t kBlock = 16;

int32_t blocks_for(int64_t tokens) { return (int32_t)((tokens + kBlock - 1) / kBlock); }
}  // namespace

struct pa_block_manager {
  int32_t num_blocks = 0;
  std::vector<int32_t> refcount;
  // Free list: a queue in a ring of num_blocks entries (a block is on it at
  // most once, so it never holds more).
  std::vector<int32_t> ring;
  int32_t head = 0, count = 0;
  std::vector<std::vector<int32_t>> tables;  // per sequence id
  std::vector<int64_t> lengths;
  std::vector<uint8_t> live;
  mutable std::mutex mu;

  int32_t take() {
    const int32_t b = ring[head];
    head = head + 1 == num_blocks ? 0 : head + 1;
    --count;
    refcount[b] = 1;
    return b;
  }
  void give_back(int32_t b) {
    int32_t tail = head + count;
    if (tail >= num_blocks) tail -= num_blocks;
    ring[tail] = b;
    ++count;
  }
  bool valid(int32_t seq) const {
    return seq >= 0 && seq < (int32_t)tables.size() && live[seq];
  }
  // Blocks an append of n tokens to seq takes: the new blocks past its last
  // one, plus one for the copy when its partly filled last block is shared.
  int32_t needed(int32_t seq, int32_t n) const {
    const int64_t C = lengths[seq];
    const int32_t fresh = blocks_for(C + n) - blocks_for(C);
    const bool cow = n > 0 && C % kBlock != 0 && refcount[tables[seq].back()] >= 2;
    return fresh + (cow ? 1 : 0);
  }
  int32_t push_sequence(std::vector<int32_t> tab, int64_t len) {
    for (int32_t b : tab) ++refcount[b];
    tables.push_back(std::move(tab));
    lengths.push_back(len);
    live.push_back(1);
    return (int32_t)tables.size() - 1;
  }
};

extern "C" {

int32_t pa_bm_create(int32_t num_blocks, const int32_t* free_order, pa_block_manager** out) {
  if (!out || num_blocks <= 0 || (int64_t)num_blocks * kBlock > INT32_MAX) return PA_EINVAL;
  *out = nullptr;
  auto* bm = new pa_block_manager;
  bm->num_blocks = num_blocks;
  bm->refcount.assign(num_blocks, 0);
  bm->ring.resize(num_blocks);
  std::vector<uint8_t> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      return PA_EINVAL;
    }
    seen[b] = 1;
    bm->ring[i] = b;
  }
  bm->count = num_blocks;
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq) {
  if (!bm || !seq) return PA_EINVAL;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (bm->tables.size() >= (size_t)INT32_MAX) return PA_EINVAL;
  *seq = bm->push_sequence({}, 0);
  return PA_OK;
}

int32_t pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child) {
  if (!bm || !child) return PA_EINVAL;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->valid(parent) || bm->tables.size() >= (size_t)INT32_MAX) return PA_EINVAL;
  *child = bm->push_sequence(bm->tables[parent], bm->lengths[parent]);
  return PA_OK;
}

int32_t pa_bm_share_prefix(pa_block_manager* bm, int32_t src, int32_t num_tokens,
                           int32_t* seq) {
  if (!bm || !seq) return PA_EINVAL;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->valid(src) || num_tokens < 0 || num_tokens > bm->lengths[src] ||
      bm->tables.size() >= (size_t)INT32_MAX)
    return PA_EINVAL;
  const std::vector<int32_t>& t = bm->tables[src];
  *seq = bm->push_sequence(std::vector<int32_t>(t.begin(), t.begin() + blocks_for(num_tokens)),
                           num_tokens);
  return PA_OK;
}

int32_t pa_bm_blocks_needed(const pa_block_manager* bm, int32_t seq, int32_t num_tokens) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->valid(seq) || num_tokens < 0 || bm->lengths[seq] + num_tokens > INT32_MAX) return -1;
  return bm->needed(seq, num_tokens);
}

int32_t pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t num_tokens, int32_t* slots,
                     int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies) {
  if (!bm || !num_copies || num_tokens < 0 || (num_tokens > 0 && !slots) ||
      !copy_src || !copy_dst)
    return PA_EINVAL;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->valid(seq) || bm->lengths[seq] + num_tokens > INT32_MAX) return PA_EINVAL;
  if (bm->needed(seq, num_tokens) > bm->count) return PA_ENOBLOCKS;
  std::vector<int32_t>& tab = bm->tables[seq];
  const int64_t C = bm->lengths[seq];
  *num_copies = 0;
  if (num_tokens > 0 && C % kBlock != 0 && bm->refcount[tab.back()] >= 2) {
    // The write would land in a block other sequences still read: copy it.
    const int32_t old = tab.back();
    const int32_t fresh = bm->take();
    --bm->refcount[old];
    tab.back() = fresh;
    *copy_src = old;
    *copy_dst = fresh;
    *num_copies = 1;
  }
  for (int64_t pos = C; pos < C + num_tokens; ++pos) {
    if (pos % kBlock == 0) tab.push_back(bm->take());
    slots[pos - C] = tab[pos / kBlock] * kBlock + (int32_t)(pos % kBlock);
  }
  bm->lengths[seq] = C + num_tokens;
  return PA_OK;
}

int32_t pa_bm_free_sequence(pa_block_manager* bm, int32_t seq) {
  if (!bm) return PA_EINVAL;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (!bm->valid(seq)) return PA_EINVAL;
  for (int32_t b : bm->tables[seq])
    if (--bm->refcount[b] == 0) bm->give_back(b);
  bm->tables[seq].clear();
  bm->tables[seq].shrink_to_fit();
  bm->lengths[seq] = 0;
  bm->live[seq] = 0;
  return PA_OK;
}

int32_t pa_bm_num_free(const pa_block_manager* bm) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return bm->count;
}

int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  if (block < 0 || block >= bm->num_blocks) return -1;
  return bm->refcount[block];
}

int32_t pa_bm_length(const pa_block_manager* bm, int32_t seq) {
  if (!bm) return -1;
  std::lock_guard<std::mutex> lock(bm->mu);
  return bm->valid(seq) ? (int32_t)bm->lengths[seq] : -1;
}

int32_t pa_bm_tables(const pa_block_manager* bm, const int32_t* seqs, int32_t num_seqs,
                     int32_t max_blocks_per_seq, int32_t* block_tables, int32_t* context_lens) {
  if (!bm || num_seqs < 0 || max_blocks_per_seq < 0) return PA_EINVAL;
  if (num_seqs > 0 && (!seqs || !context_lens || (max_blocks_per_seq > 0 && !block_tables)))
    return PA_EINVAL;
  std::lock_guard<std::mutex> lock(bm->mu);
  for (int32_t i = 0; i < num_seqs; ++i)
    if (!bm->valid(seqs[i]) || (int64_t)bm->tables[seqs[i]].size() > max_blocks_per_seq)
      return PA_EINVAL;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const std::vector<int32_t>& t = bm->tables[seqs[i]];
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < (int32_t)t.size() ? t[j] : -1;
    context_lens[i] = (int32_t)bm->lengths[seqs[i]];
  }
  return PA_OK;
}

}  // extern "C"

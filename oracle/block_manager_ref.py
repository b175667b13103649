"""Plain CPU model of paged KV block management -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` import this module; the product path (libpa's host block
manager and its copy kernel) never calls it and shares no code with it.

What it models, and where the pages define it:

* Every sequence owns a block table mapping its logical blocks to physical
  blocks of a shared pool of 16-token blocks (SOSP 2023 PagedAttention
  explainer, "ブロックテーブルによるメモリ管理").
* Appending a token writes it into the sequence's current physical block
  while that block has room, and into a block newly taken from the free list
  once it is full; a finished sequence returns its blocks to the free list at
  once (same section).  So a sequence of C tokens holds ceil(C / 16) blocks
  and wastes at most B - 1 slots, all in its last block.
* Sequences share a physical block by holding the same table entry: parallel
  samples of one prompt share the prompt's blocks, and a request whose prefix
  matches an earlier one shares that prefix's blocks ("Copy-on-Writeによる
  メモリ共有", "Prefix Caching").  Every physical block carries a reference
  count; a write into a block whose count is 2 or more first copies the block
  and writes into the copy (copy-on-write, same section).  Since appends only
  ever write at a sequence's end, the one block a write can hit is the
  sequence's partly filled last block.
* ``copy_blocks_ref`` is the copy itself on raw 16-bit patterns: every K and V
  row of block ``dst[i]`` becomes those of block ``src[i]``.
* ``swap_blocks_ref`` is the same copy between two pools: KV evicted from the
  GPU lives in a CPU tier of blocks and is copied back before the layer that
  reads it runs (Pensieve explainer, "GPU-CPU 2層キャッシュ構造",
  "パイプライン化されたswap-in").

Policy choices the pages leave open (the library's manager takes the same
ones, as a convention, not as code): the free list is a queue, taken from the
front and returned to the back, with a caller-given initial order; a block
freed by a sequence goes back in table order; the copy of a copy-on-write is
taken from the free list before any new block of the same append; sequence
ids count up from 0 and are never reused.
"""
from __future__ import annotations

from collections import deque

import numpy as np

BLOCK = 16


class BlockManagerRef:
    """Free list, reference counts and per-sequence block tables."""

    def __init__(self, num_blocks: int, free_order=None):
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        assert sorted(order) == list(range(num_blocks)), "free_order must list every block once"
        self.num_blocks = num_blocks
        self.free = deque(order)
        self.refcount = [0] * num_blocks
        self.tables = []   # per sequence id: list of physical blocks, or None once freed
        self.lengths = []  # per sequence id: tokens held

    # -- queries ---------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def live(self, seq: int) -> bool:
        return 0 <= seq < len(self.tables) and self.tables[seq] is not None

    def table(self, seq: int):
        assert self.live(seq), "no such sequence"
        return list(self.tables[seq])

    def length(self, seq: int) -> int:
        assert self.live(seq), "no such sequence"
        return self.lengths[seq]

    # -- operations ------------------------------------------------------
    def _take(self) -> int:
        b = self.free.popleft()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def add_sequence(self) -> int:
        self.tables.append([])
        self.lengths.append(0)
        return len(self.tables) - 1

    def fork(self, parent: int) -> int:
        """A new sequence holding the parent's tokens in the parent's blocks."""
        tab = self.table(parent)
        for b in tab:
            self.refcount[b] += 1
        self.tables.append(tab)
        self.lengths.append(self.lengths[parent])
        return len(self.tables) - 1

    def share_prefix(self, src: int, num_tokens: int) -> int:
        """A new sequence holding the first num_tokens tokens of src, in src's
        first ceil(num_tokens / 16) blocks."""
        assert 0 <= num_tokens <= self.length(src)
        tab = self.table(src)[: -(-num_tokens // BLOCK)]
        for b in tab:
            self.refcount[b] += 1
        self.tables.append(tab)
        self.lengths.append(num_tokens)
        return len(self.tables) - 1

    def blocks_needed(self, seq: int, num_tokens: int) -> int:
        """Blocks an append of num_tokens would take from the free list."""
        C = self.length(seq)
        new = -(-(C + num_tokens) // BLOCK) - (-(-C // BLOCK))
        cow = num_tokens > 0 and C % BLOCK != 0 and self.refcount[self.tables[seq][-1]] >= 2
        return new + (1 if cow else 0)

    def append(self, seq: int, num_tokens: int):
        """Room for num_tokens new tokens at the sequence's end.

        Returns (slots, copies): the slot (block * 16 + offset) of each new
        token in order, and the (src, dst) block copies that must happen
        before the new tokens are written.  Raises MemoryError, changing
        nothing, when the free list is too short.
        """
        assert num_tokens >= 0
        if self.blocks_needed(seq, num_tokens) > len(self.free):
            raise MemoryError("free list exhausted")
        tab = self.tables[seq]
        C = self.lengths[seq]
        copies = []
        if num_tokens > 0 and C % BLOCK != 0 and self.refcount[tab[-1]] >= 2:
            old = tab[-1]
            new = self._take()
            self.refcount[old] -= 1
            tab[-1] = new
            copies.append((old, new))
        slots = []
        for pos in range(C, C + num_tokens):
            if pos % BLOCK == 0:
                tab.append(self._take())
            slots.append(tab[pos // BLOCK] * BLOCK + pos % BLOCK)
        self.lengths[seq] = C + num_tokens
        return slots, copies

    def free_sequence(self, seq: int) -> None:
        """The sequence is done: each of its blocks loses a reference, and a
        block nobody references goes back to the free list."""
        for b in self.table(seq):
            self.refcount[b] -= 1
            assert self.refcount[b] >= 0
            if self.refcount[b] == 0:
                self.free.append(b)
        self.tables[seq] = None
        self.lengths[seq] = 0

    def tables_array(self, seqs, max_blocks: int):
        """[len(seqs), max_blocks] int32 tables (padding -1) and int32 lengths."""
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            tab = self.table(s)
            assert len(tab) <= max_blocks
            out[i, :len(tab)] = tab
            lens[i] = self.lengths[s]
        return out, lens


def copy_blocks_ref(k_pool: np.ndarray, v_pool: np.ndarray, src, dst):
    """Copies of (k_pool, v_pool) ``[NB, Hkv, 16, D]`` (16-bit patterns) in which
    block dst[i] holds block src[i]'s K and V rows.  dst blocks are distinct
    and none of them is a src block, so the copies are independent."""
    src = [int(x) for x in src]
    dst = [int(x) for x in dst]
    assert len(src) == len(dst)
    assert len(set(dst)) == len(dst), "a block is copied into twice"
    assert not set(dst) & set(src), "a copy's destination is another copy's source"
    k_out = np.array(k_pool, dtype=np.uint16, copy=True)
    v_out = np.array(v_pool, dtype=np.uint16, copy=True)
    for s, d in zip(src, dst):
        k_out[d] = k_pool[s]
        v_out[d] = v_pool[s]
    return k_out, v_out


def swap_blocks_ref(dst_k: np.ndarray, dst_v: np.ndarray, src_k: np.ndarray,
                    src_v: np.ndarray, src_ids, dst_ids):
    """Copies of the destination pools in which block dst_ids[i] holds block
    src_ids[i] of the source pools (16-bit patterns, same block shape)."""
    src_ids = [int(x) for x in src_ids]
    dst_ids = [int(x) for x in dst_ids]
    assert len(src_ids) == len(dst_ids)
    assert len(set(dst_ids)) == len(dst_ids), "a block is copied into twice"
    assert dst_k.shape[1:] == src_k.shape[1:]
    k_out = np.array(dst_k, dtype=np.uint16, copy=True)
    v_out = np.array(dst_v, dtype=np.uint16, copy=True)
    for s, d in zip(src_ids, dst_ids):
        k_out[d] = src_k[s]
        v_out[d] = src_v[s]
    return k_out, v_out

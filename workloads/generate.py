"""Seeded synthetic inputs for generalized paged attention.

This module only *produces inputs*: query rows, physical K/V pools, block
tables, context lengths, query offsets and slot mappings.  It holds none of
the attention arithmetic, so both the CPU oracle (``oracle/``) and the HIP
path consume exactly the same bits without sharing any method code.

Conventions (the pages fix only the 16-token block and the per-sequence
block table, PagedAttention explainer, "ブロックテーブルによるメモリ管理"):

* dtype ``"f16"`` or ``"bf16"``; tensors of that dtype are stored here as
  ``uint16`` bit patterns.  Values are drawn N(0, 1) in float32 and rounded
  once (round-to-nearest-even) to the 16-bit type.
* pools are ``[num_blocks, num_kv_heads, block_size, head_dim]``.
* ``context_lens[s]`` counts every key sequence ``s`` can see, including its
  ``n_s`` new tokens; the new tokens occupy positions ``C_s - n_s .. C_s - 1``.
* the new tokens' K/V are *not* in the pool yet: their slots hold a poison
  pattern (NaN) until ``pa_kv_write`` scatters ``k_new``/``v_new`` there.
  Every other slot that no sequence may read (free blocks, the tail of a
  partial last block) also holds NaN, so an out-of-range read shows up.
* block-table entries past a sequence's last block are padding (``-1`` by
  default) and must never be dereferenced.
* ``slot = physical_block * block_size + offset``; ``-1`` means "skip".
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
HEAD_DIM = 128

# Quiet-NaN bit patterns used to poison slots that must never be read.
POISON = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def _round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> 16-bit pattern of ``dtype`` with round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32)
        return ((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def _worker_count() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bits(seed_seq: np.random.SeedSequence, shape, dtype: str,
                chunk: int = 1 << 22) -> np.ndarray:
    """N(0,1) values of ``shape`` as 16-bit patterns.

    The flat array is cut into fixed chunks, each drawn from its own child of
    ``seed_seq``; the result depends only on the seed, never on how many
    threads filled it.
    """
    total = int(np.prod(shape, dtype=np.int64))
    out = np.empty(total, dtype=np.uint16)
    nchunks = max(1, -(-total // chunk))
    children = seed_seq.spawn(nchunks)

    def fill(i: int) -> None:
        lo = i * chunk
        hi = min(total, lo + chunk)
        rng = np.random.default_rng(children[i])
        out[lo:hi] = _round_bits(rng.standard_normal(hi - lo, dtype=np.float32), dtype)

    if nchunks == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_worker_count()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclass
class PagedWorkload:
    """One layer's worth of paged-attention inputs (all host arrays)."""

    name: str
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    q: np.ndarray              # uint16 [Tq, Hq, D]
    k_pool: np.ndarray         # uint16 [NB, Hkv, B, D]   state before pa_kv_write
    v_pool: np.ndarray         # uint16 [NB, Hkv, B, D]
    k_new: np.ndarray          # uint16 [T, Hkv, D]
    v_new: np.ndarray          # uint16 [T, Hkv, D]
    slot_mapping: np.ndarray   # int32 [T]
    block_tables: np.ndarray   # int32 [S, max_blocks]
    context_lens: np.ndarray   # int32 [S]
    query_start_loc: np.ndarray  # int32 [S+1]
    refcounts: np.ndarray      # int32 [NB]  how many tables reference each block
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start_loc).astype(np.int64)

    @property
    def max_query_len(self) -> int:
        ql = self.query_lens
        return int(ql.max()) if ql.size else 0

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])


def blocks_for(tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Blocks needed to hold ``tokens`` tokens (allocation size)."""
    return -(-int(tokens) // block_size)


def build_workload(name: str, seed, *, dtype: str, num_q_heads: int, num_kv_heads: int,
                   cached_lens, new_lens, pool_factor: float = 1.2,
                   num_blocks: int | None = None, placement: str = "shuffled",
                   shared_prefix_groups=None, shared_prefix_blocks: int = 0,
                   head_dim: int = HEAD_DIM, block_size: int = BLOCK_SIZE,
                   scale: float | None = None, table_pad: int = -1,
                   extra_table_cols: int = 0, new_in_pool=False) -> PagedWorkload:
    """Build a seeded workload.

    ``cached_lens[s]`` tokens of sequence ``s`` are already in the pool;
    ``new_lens[s]`` new tokens follow them and are the sequence's query rows.
    ``new_in_pool`` (a bool, or one bool per sequence) marks sequences whose
    new tokens' K/V are already in the pool as ordinary cached data: their
    ``slot_mapping`` entries are ``-1`` (skip) and their ``k_new``/``v_new``
    rows are never used.  This is how a sample whose newest key sits in a
    shared prefix block is expressed: nothing may be written there.

    ``shared_prefix_groups``: list of lists of sequence indices; the members
    of one group share their first ``shared_prefix_blocks`` physical blocks
    (identical block-table entries, refcount = group size).  Shared blocks
    must hold only cached tokens.

    ``placement``: ``"shuffled"`` pops blocks in order from a random
    permutation of the pool (a shuffled free list); ``"contiguous"`` hands out
    blocks 0, 1, 2, ... in order.
    """
    ss = np.random.SeedSequence(seed)
    ss_meta, ss_q, ss_k, ss_v, ss_kn, ss_vn = ss.spawn(6)
    rng = np.random.default_rng(ss_meta)

    cached = np.asarray(cached_lens, dtype=np.int64)
    new = np.asarray(new_lens, dtype=np.int64)
    assert cached.shape == new.shape and cached.ndim == 1
    S = cached.shape[0]
    C = cached + new
    nblk = np.array([blocks_for(c, block_size) for c in C], dtype=np.int64)

    in_pool = np.broadcast_to(np.asarray(new_in_pool, dtype=bool), (S,))
    share_of = {}
    groups = [list(g) for g in (shared_prefix_groups or [])]
    for gi, g in enumerate(groups):
        for s in g:
            assert s not in share_of
            share_of[s] = gi
            pooled = cached[s] + (new[s] if in_pool[s] else 0)
            assert pooled >= shared_prefix_blocks * block_size, \
                "shared prefix blocks must hold cached tokens only"
            assert nblk[s] >= shared_prefix_blocks
    need = int(nblk.sum()) - sum((len(g) - 1) * shared_prefix_blocks for g in groups)
    NB = int(num_blocks) if num_blocks is not None else int(math.ceil(pool_factor * need))
    assert NB >= need, "pool too small"

    if placement == "shuffled":
        free = [int(b) for b in rng.permutation(NB)]
    elif placement == "contiguous":
        free = list(range(NB))
    else:
        raise ValueError(placement)
    free.reverse()  # pop() hands out the permutation in order

    max_blocks = int(nblk.max()) + extra_table_cols if S else 1
    tables = np.full((S, max(1, max_blocks)), table_pad, dtype=np.int32)
    refc = np.zeros(NB, dtype=np.int32)
    group_prefix = {}
    for s in range(S):
        row = []
        gi = share_of.get(s)
        if gi is not None:
            if gi not in group_prefix:
                group_prefix[gi] = [free.pop() for _ in range(shared_prefix_blocks)]
            row.extend(group_prefix[gi])
        while len(row) < nblk[s]:
            row.append(free.pop())
        tables[s, :nblk[s]] = row
        for b in row:
            refc[b] += 1

    Hkv, D, B = num_kv_heads, head_dim, block_size
    poison = POISON[dtype]
    k_pool = np.full((NB, Hkv, B, D), poison, dtype=np.uint16)
    v_pool = np.full((NB, Hkv, B, D), poison, dtype=np.uint16)

    # Fresh N(0,1) K/V for every referenced block, drawn in physical order.
    used = np.flatnonzero(refc > 0)
    k_pool[used] = normal_bits(ss_k, (used.size, Hkv, B, D), dtype)
    v_pool[used] = normal_bits(ss_v, (used.size, Hkv, B, D), dtype)

    # Slots at or past each sequence's visible length hold poison; so do the
    # slots of new tokens (until pa_kv_write) unless new_in_pool.
    T = int(new.sum())
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(new)
    k_new = normal_bits(ss_kn, (T, Hkv, D), dtype)
    v_new = normal_bits(ss_vn, (T, Hkv, D), dtype)
    slots = np.full(T, -1, dtype=np.int32)
    for s in range(S):
        row = tables[s]
        last = int(nblk[s]) - 1
        tail_from = int(C[s]) - last * B
        if tail_from < B:
            blk = int(row[last])
            assert refc[blk] == 1 or C[s] % B == 0
            k_pool[blk, :, tail_from:, :] = poison
            v_pool[blk, :, tail_from:, :] = poison
        for i in range(int(new[s])):
            pos = int(cached[s]) + i
            blk = int(row[pos // B])
            off = pos % B
            t = int(qsl[s]) + i
            if in_pool[s]:
                continue  # the key is already cached; nothing to write
            assert refc[blk] == 1, "new tokens must land in private blocks"
            k_pool[blk, :, off, :] = poison
            v_pool[blk, :, off, :] = poison
            slots[t] = blk * B + off

    q = normal_bits(ss_q, (T, num_q_heads, D), dtype)
    return PagedWorkload(
        name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=D, block_size=B,
        scale=float(scale) if scale is not None else 1.0 / math.sqrt(D),
        q=q, k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, slot_mapping=slots,
        block_tables=tables, context_lens=C.astype(np.int32), query_start_loc=qsl,
        refcounts=refc,
        meta={"cached_lens": cached, "new_lens": new, "pool_need": need,
              "placement": placement, "seed": seed})

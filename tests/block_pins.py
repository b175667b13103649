"""Checks that tie the block-management model of the oracle to the pages.

Each ``pin_*`` takes the model's module (``oracle.block_manager_ref`` or a
copy with a planted mistake) and raises ``AssertionError`` when it disagrees
with the pages' worked example, a closed form, a conservation law, or the
one property block sharing must keep: every live sequence reads back exactly
the tokens it was given, whatever the other sequences write.
"""
from __future__ import annotations

import json
import os

import numpy as np

B = 16
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pin_page_block_tables(o):
    """The explainer's figures: A holds [7, 1, 3]; B shares A's first two
    blocks and owns 5; blocks 7 and 1 have reference count 2.  A third
    sequence sharing all of A's 40 tokens, then writing its 41st, makes the
    write hit block 3 (count 2): block 3 is copied first."""
    with open(os.path.join(GOLDEN, "block_table_example.json")) as f:
        ex = json.load(f)
    free = [7, 1, 3, 5, 0, 2, 4, 6]
    bm = o.BlockManagerRef(ex["pool_blocks"], free)
    a = bm.add_sequence()
    slots, copies = bm.append(a, 40)
    assert bm.table(a) == ex["table_a"] and copies == []
    assert slots[0] == 7 * B and slots[16] == 1 * B and slots[39] == 3 * B + 7
    b = bm.share_prefix(a, 32)
    _, copies = bm.append(b, 8)
    assert bm.table(b) == ex["table_b"] and copies == []
    for blk in ex["shared_blocks"]:
        assert bm.refcount[blk] == ex["refcount_shared"]
    assert bm.refcount[3] == 1 and bm.refcount[5] == 1
    c = bm.share_prefix(a, 40)
    assert bm.table(c) == [7, 1, 3] and bm.refcount[3] == 2
    slots, copies = bm.append(c, 1)
    assert copies == [(3, 0)], copies
    assert bm.table(c) == [7, 1, 0] and slots == [0 * B + 8]
    assert bm.refcount[3] == 1 and bm.refcount[0] == 1 and bm.table(a) == [7, 1, 3]


def pin_fragmentation_bound(o):
    """A sequence of C tokens holds ceil(C / 16) blocks: at most B - 1 unused
    slots, all in its last block."""
    bm = o.BlockManagerRef(400, np.random.default_rng(1).permutation(400))
    rng = np.random.default_rng(2)
    seqs = [bm.add_sequence() for _ in range(12)]
    for _ in range(60):
        s = seqs[int(rng.integers(len(seqs)))]
        bm.append(s, int(rng.integers(0, 40)))
        for t in seqs:
            C = bm.length(t)
            waste = len(bm.table(t)) * B - C
            assert 0 <= waste <= B - 1 and len(bm.table(t)) == -(-C // B), (C, bm.table(t))


def _random_ops(o, seed, num_blocks=96, steps=400):
    """Random adds, forks, prefix shares, appends and frees on a token-id pool.

    Each new token gets a unique id, written at its slot after the append's
    copies are applied; after every step every live sequence must read back,
    through its table, exactly the ids it was given.  Yields the manager after
    each step for further checks.
    """
    rng = np.random.default_rng(seed)
    bm = o.BlockManagerRef(num_blocks, rng.permutation(num_blocks))
    pool = np.full((num_blocks, B), -1, dtype=np.int64)
    content = {}
    next_id = 0
    for _ in range(steps):
        live = [s for s in content]
        op = rng.integers(0, 10)
        if op == 0 or not live:
            s = bm.add_sequence()
            content[s] = []
        elif op == 1:
            p = live[int(rng.integers(len(live)))]
            content[bm.fork(p)] = list(content[p])
        elif op == 2:
            p = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, len(content[p]) + 1))
            content[bm.share_prefix(p, n)] = content[p][:n]
        elif op == 3 and len(live) > 1:
            s = live[int(rng.integers(len(live)))]
            bm.free_sequence(s)
            del content[s]
        else:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(1, 24))
            before = (bm.num_free(), list(bm.refcount), bm.table(s))
            try:
                slots, copies = bm.append(s, n)
            except MemoryError:
                assert (bm.num_free(), list(bm.refcount), bm.table(s)) == before, \
                    "a failed append changed the manager"
                yield bm, content, pool
                continue
            for src, dst in copies:
                pool[dst] = pool[src]
            for slot in slots:
                pool[slot // B, slot % B] = next_id
                content[s].append(next_id)
                next_id += 1
        for s, toks in content.items():
            tab = bm.table(s)
            got = [int(pool[tab[i // B], i % B]) for i in range(len(toks))]
            assert got == toks, f"sequence {s} reads {got[:8]}.. instead of {toks[:8]}.."
        yield bm, content, pool


def pin_sharing_keeps_every_sequence_intact(o):
    """Forks, shared prefixes and appends in random order: every live
    sequence reads back its own tokens (copy-on-write before any write into a
    block another sequence references; no block reused while referenced)."""
    for seed in (3, 4, 5):
        for _ in _random_ops(o, seed):
            pass


def pin_reference_counts_are_conserved(o):
    """Each block's count equals the table entries naming it; a block is on
    the free list exactly when its count is 0, and at most once."""
    for bm, content, _ in _random_ops(o, 6, steps=300):
        counts = np.zeros(bm.num_blocks, dtype=np.int64)
        for s in content:
            for blk in bm.table(s):
                counts[blk] += 1
        assert list(counts) == list(bm.refcount)
        free = list(bm.free)
        assert len(set(free)) == len(free)
        assert set(free) == {b for b in range(bm.num_blocks) if bm.refcount[b] == 0}


def pin_exhausted_free_list(o):
    """An append that needs more blocks than are free fails and changes nothing."""
    bm = o.BlockManagerRef(3)
    s = bm.add_sequence()
    bm.append(s, 40)
    try:
        bm.append(s, 9)
    except MemoryError:
        pass
    else:
        raise AssertionError("append past the free list succeeded")
    assert bm.length(s) == 40 and bm.table(s) == [0, 1, 2] and bm.num_free() == 0
    bm.append(s, 8)  # fills the last block exactly: no new block needed
    assert bm.length(s) == 48


def pin_copy_blocks(o):
    """Block dst[i] gets block src[i]'s K and V bits; nothing else moves."""
    rng = np.random.default_rng(9)
    kp = rng.integers(0, 65536, size=(10, 3, B, 8), dtype=np.uint16)
    vp = rng.integers(0, 65536, size=(10, 3, B, 8), dtype=np.uint16)
    src, dst = [4, 0, 7], [2, 9, 5]
    k2, v2 = o.copy_blocks_ref(kp, vp, src, dst)
    for s, d in zip(src, dst):
        assert np.array_equal(k2[d], kp[s]) and np.array_equal(v2[d], vp[s])
    for b in set(range(10)) - set(dst):
        assert np.array_equal(k2[b], kp[b]) and np.array_equal(v2[b], vp[b])


def pin_swap_round_trip(o):
    """Blocks sent to a second pool and back, under other ids, return bit for
    bit; blocks outside the lists stay as they were in both pools."""
    rng = np.random.default_rng(10)
    gk = rng.integers(0, 65536, size=(12, 2, B, 8), dtype=np.uint16)
    gv = rng.integers(0, 65536, size=(12, 2, B, 8), dtype=np.uint16)
    hk = rng.integers(0, 65536, size=(20, 2, B, 8), dtype=np.uint16)
    hv = rng.integers(0, 65536, size=(20, 2, B, 8), dtype=np.uint16)
    out_src, out_dst = [3, 7, 0], [19, 2, 11]
    hk2, hv2 = o.swap_blocks_ref(hk, hv, gk, gv, out_src, out_dst)
    for s, d in zip(out_src, out_dst):
        assert np.array_equal(hk2[d], gk[s]) and np.array_equal(hv2[d], gv[s])
    for b in set(range(20)) - set(out_dst):
        assert np.array_equal(hk2[b], hk[b]) and np.array_equal(hv2[b], hv[b])
    back = [5, 9, 1]
    gk2, gv2 = o.swap_blocks_ref(gk, gv, hk2, hv2, out_dst, back)
    for s, d in zip(out_src, back):
        assert np.array_equal(gk2[d], gk[s]) and np.array_equal(gv2[d], gv[s])
    for b in set(range(12)) - set(back):
        assert np.array_equal(gk2[b], gk[b]) and np.array_equal(gv2[b], gv[b])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

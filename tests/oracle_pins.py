"""Checks that tie the CPU oracle to something other than itself.

Each ``pin_*`` takes the oracle module and raises ``AssertionError`` when the
oracle disagrees with a hand-derived value, a closed form, a library routine
or an invariance the mathematics fixes.  ``test_oracle_pins.py`` runs them
on the oracle as it is; ``test_oracle_mutations.py`` plants plausible
mistakes in a copy of the oracle and checks some pin catches each one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from helpers import B, brute_force, from_f64, paged_layout, random_case, to_f64
from workloads import build_workload

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _attn(o, case, scale, **kw):
    return o.attention_ref(case["q"], case["k_pool"], case["v_pool"], case["block_tables"],
                           case["context_lens"], case["query_start_loc"], case["num_kv_heads"],
                           scale, case["dtype"], **kw)


def _single(o, q_rows, k_rows, v_rows, scale, dtype="f16", n=None, seed=0):
    """One sequence, one head, D = len(q_rows[0]); exact inputs; returns [n, D]."""
    q = from_f64(np.asarray(q_rows, dtype=np.float64), dtype)[:, None, :]
    K = from_f64(np.asarray(k_rows, dtype=np.float64), dtype)[:, None, :]
    V = from_f64(np.asarray(v_rows, dtype=np.float64), dtype)[:, None, :]
    C = K.shape[0]
    n = q.shape[0] if n is None else n
    nb = -(-C // B) + 2
    kp, vp, tab = paged_layout([K], [V], nb, np.random.default_rng(seed))
    out, _ = o.attention_ref(q, kp, vp, tab, np.array([C], np.int32),
                             np.array([0, n], np.int32), 1, scale, dtype)
    return out[:, 0, :]


# --------------------------------------------------------------------------
# hand-derived values
# --------------------------------------------------------------------------
def pin_two_key_softmax(o):
    """Logits 0 and 1 (after scale) give weights 1/(1+e) and e/(1+e)."""
    q = [[1.0, 0.0, 0.0, 0.0]]
    k = [[0.0, 0.0, 0.0, 0.0], [2.0, 0.0, 0.0, 0.0]]
    v = [[1.0, 0.0, 4.0, -2.0], [0.0, 1.0, 2.0, 8.0]]
    got = _single(o, q, k, v, scale=0.5)[0]
    e = math.e
    want = (np.array(v[0]) + e * np.array(v[1])) / (1 + e)
    assert np.max(np.abs(got - want)) <= 1e-14, (got, want)


def pin_query_key_orientation(o):
    """Logit of key j is <q, k_j> (not <k_0, q_j> etc.): distinct keys, one query."""
    q = [[0.0, 1.0, 0.0, 0.0]]
    k = [[1.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0], [0.0, 2.0, 0.0, 0.0]]
    v = [[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0], [0.0, 0.0, 1.0, 0.0]]
    got = _single(o, q, k, v, scale=1.0)[0]
    w = np.array([1.0, 1.0, math.exp(2.0)])
    want = w / w.sum()
    assert np.max(np.abs(got[:3] - want)) <= 1e-14 and got[3] == 0.0, (got, want)


def pin_bottom_right_causal(o):
    """n = 2 new rows over C = 3 keys, q = 0: row 0 averages keys 0..1, row 1 keys 0..2."""
    q = [[0.0] * 4, [0.0] * 4]
    k = [[1.0, 2.0, 3.0, 4.0], [-1.0, 0.5, 2.0, 0.0], [0.25, -3.0, 1.0, 1.0]]
    v = [[3.0, 0.0, 1.0, 2.0], [1.0, 6.0, -1.0, 4.0], [2.0, 3.0, 9.0, -6.0]]
    got = _single(o, q, k, v, scale=0.7)
    V = np.array(v)
    assert np.max(np.abs(got[0] - V[:2].mean(0))) <= 1e-14, got
    assert np.max(np.abs(got[1] - V[:3].mean(0))) <= 1e-14, got


def pin_single_key(o):
    """C = 1: the output is v_0 exactly, whatever q and the scale."""
    rng = np.random.default_rng(7)
    for dtype in ("f16", "bf16"):
        for _ in range(5):
            q = rng.standard_normal((1, 8)).astype(np.float16).astype(np.float64)
            k = rng.standard_normal((1, 8)).astype(np.float16).astype(np.float64)
            v = rng.integers(-8, 8, size=(1, 8)).astype(np.float64)
            if dtype == "bf16":
                q = np.round(q * 4) / 4
                k = np.round(k * 4) / 4
            got = _single(o, q, k, v, scale=0.3, dtype=dtype)
            assert np.array_equal(got[0], v[0]), (got, v)


def pin_dominant_key(o):
    """One logit 60 above the rest: the output is that key's v to 1e-12."""
    D = 8
    q = np.zeros((1, D)); q[0, 0] = 4.0
    k = np.zeros((37, D)); k[21, 0] = 15.0  # logit 60 at key 21, 0 elsewhere
    v = np.arange(37 * D, dtype=np.float64).reshape(37, D) % 17 - 8
    got = _single(o, q, k, v, scale=1.0)[0]
    assert np.max(np.abs(got - v[21])) <= 1e-12 * np.abs(v).max(), got


def pin_equal_keys_mean(o):
    """All visible keys equal: weights are uniform, output = mean of visible V."""
    D = 8
    rng = np.random.default_rng(3)
    C, n = 45, 5
    k = np.tile(np.array([[0.5, -1.0, 2.0, 0.0, 1.0, 0.25, -0.5, 3.0]]), (C, 1))
    v = rng.integers(-16, 16, size=(C, D)).astype(np.float64)
    q = rng.integers(-2, 3, size=(n, D)).astype(np.float64)
    got = _single(o, q, k, v, scale=0.125)
    for i in range(n):
        visible = C - n + i + 1
        assert np.max(np.abs(got[i] - v[:visible].mean(0))) <= 1e-12, i


# --------------------------------------------------------------------------
# library routine / brute force over contiguous K, V
# --------------------------------------------------------------------------
TINY_CASES = [
    # (seed, contexts, new tokens, Hq, Hkv, dtype)
    (11, [1], [1], 2, 2, "f16"),
    (12, [16, 17, 70], [16, 3, 0], 4, 2, "f16"),
    (13, [33, 5, 48], [1, 5, 48], 4, 1, "bf16"),
    (14, [31, 64], [7, 2], 8, 2, "bf16"),
    (15, [69], [30], 4, 4, "f16"),
]


def pin_brute_force_sdpa(o):
    """Paged gather + softmax equals torch SDPA (CPU fp64) over contiguous K/V."""
    for seed, ctx, new, hq, hkv, dtype in TINY_CASES:
        case = random_case(seed, ctx, new, hq, hkv, dtype)
        scale = 1.0 / math.sqrt(128)
        got, _ = _attn(o, case, scale)
        want = brute_force(case["q"], case["lk"], case["lv"], ctx, case["query_start_loc"],
                           hkv, scale, dtype)
        assert np.max(np.abs(got - want)) <= 1e-12, (seed, np.max(np.abs(got - want)))


# Batches with empty sequences (repeated query_start_loc entries) at the
# start, middle and end, so that mapping a token to its sequence must skip them.
SAMPLE_CASES = [
    # (seed, contexts, new tokens, Hq, Hkv, dtype)
    (21, [5, 16, 9, 40], [0, 3, 0, 7], 4, 2, "f16"),
    (22, [33, 1, 20, 18], [1, 1, 20, 0], 2, 1, "bf16"),
    (23, [7, 64, 0, 3], [7, 2, 0, 3], 8, 4, "f16"),
]


def pin_sample_rows(o):
    """attention_ref_sample at every (token, head), first and last rows of
    each sequence included, equals brute force over contiguous K/V."""
    for seed, ctx, new, hq, hkv, dtype in SAMPLE_CASES:
        case = random_case(seed, ctx, new, hq, hkv, dtype)
        scale = 1.0 / math.sqrt(128)
        Tq = case["q"].shape[0]
        picks = [(t, h) for t in range(Tq) for h in range(hq)]
        got = o.attention_ref_sample(case["q"], case["k_pool"], case["v_pool"],
                                     case["block_tables"], case["context_lens"],
                                     case["query_start_loc"], hkv, scale, dtype, picks)
        want = brute_force(case["q"], case["lk"], case["lv"], ctx, case["query_start_loc"],
                           hkv, scale, dtype)
        sel = np.stack([want[t, h] for t, h in picks])
        assert got.shape == sel.shape
        assert np.max(np.abs(got - sel)) <= 1e-12, (seed, np.max(np.abs(got - sel)))


def pin_blockwise_equals(o):
    """The per-block equation and the plain definition agree to 1e-12."""
    for seed, ctx, new, hq, hkv, dtype in TINY_CASES[1:4]:
        case = random_case(seed, ctx, new, hq, hkv, dtype)
        scale = 1.0 / math.sqrt(128)
        a, _ = _attn(o, case, scale)
        b = o.attention_blockwise_ref(case["q"], case["k_pool"], case["v_pool"],
                                      case["block_tables"], case["context_lens"],
                                      case["query_start_loc"], hkv, scale, dtype)
        assert np.max(np.abs(a - b)) <= 1e-12


def pin_split_merge_equals(o):
    """Any partition of the keys, merged, equals the plain result to 1e-12."""
    case = random_case(21, [70, 40], [6, 40], 4, 2, "f16")
    scale = 1.0 / math.sqrt(128)
    want, want_lse = _attn(o, case, scale)
    rng = np.random.default_rng(99)
    for trial in range(100):
        def cuts(s, h, i, visible, rng=rng):
            k = int(rng.integers(0, min(6, visible)))
            return sorted(rng.choice(np.arange(1, visible), size=k, replace=False)) if k else []
        got, lse = o.attention_split_merge_ref(
            case["q"], case["k_pool"], case["v_pool"], case["block_tables"],
            case["context_lens"], case["query_start_loc"], 2, scale, "f16", cuts)
        assert np.max(np.abs(got - want)) <= 1e-12, trial
        assert np.max(np.abs(lse - want_lse)) <= 1e-12, trial


def pin_merge_two_partitions_closed_form(o):
    """Two one-key partitions with logits a, b merge to softmax weights of (a, b)."""
    va, vb = np.array([1.0, -2.0]), np.array([4.0, 0.5])
    a, b = 0.3, -1.2
    parts = [o.partition_state(np.array([a]), va[None]), o.partition_state(np.array([b]), vb[None])]
    out, lse = o.merge_partitions(parts)
    wa = math.exp(a) / (math.exp(a) + math.exp(b))
    assert np.max(np.abs(out - (wa * va + (1 - wa) * vb))) <= 1e-15
    assert abs(lse - math.log(math.exp(a) + math.exp(b))) <= 1e-15


# --------------------------------------------------------------------------
# invariances and identities
# --------------------------------------------------------------------------
def pin_softmax_rows(o):
    """Weights are >= 0, sum to 1 per row, and are exactly 0 on masked keys."""
    case = random_case(31, [50, 23], [9, 23], 4, 2, "bf16")
    _, _, W = _attn(o, case, 0.088, return_weights=True)
    qsl = case["query_start_loc"]
    for (s, h), w in W.items():
        n, C = int(qsl[s + 1] - qsl[s]), int(case["context_lens"][s])
        assert w.shape == (n, C)
        assert np.all(w >= 0)
        assert np.max(np.abs(w.sum(1) - 1.0)) <= 1e-12
        for i in range(n):
            assert np.all(w[i, C - n + i + 1:] == 0.0)
            assert np.all(w[i, :C - n + i + 1] > 0.0)


def pin_permutation_invariance(o):
    """Relabelling physical blocks (pool and tables together) changes no bit."""
    wl = build_workload("perm", 41, dtype="f16", num_q_heads=4, num_kv_heads=2,
                        cached_lens=[40, 17, 3], new_lens=[3, 4, 1], pool_factor=2.0,
                        new_in_pool=True)
    base, _ = o.attention_ref(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                              wl.query_start_loc, wl.num_kv_heads, wl.scale, wl.dtype)
    rng = np.random.default_rng(5)
    for _ in range(3):
        pi = rng.permutation(wl.num_blocks)
        kp = np.empty_like(wl.k_pool); vp = np.empty_like(wl.v_pool)
        kp[pi] = wl.k_pool; vp[pi] = wl.v_pool
        tab = np.where(wl.block_tables >= 0, pi[np.maximum(wl.block_tables, 0)], -1).astype(np.int32)
        got, _ = o.attention_ref(wl.q, kp, vp, tab, wl.context_lens, wl.query_start_loc,
                                 wl.num_kv_heads, wl.scale, wl.dtype)
        assert np.array_equal(got, base)


def pin_shared_prefix_invariance(o):
    """Sequences sharing prefix blocks give the same output as private copies."""
    wl = build_workload("cow", 42, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                        cached_lens=[63, 70, 47, 48], new_lens=[1, 1, 1, 1], pool_factor=1.5,
                        shared_prefix_groups=[[0, 1, 2, 3]], shared_prefix_blocks=3,
                        new_in_pool=True)
    assert wl.refcounts.max() == 4
    base, _ = o.attention_ref(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                              wl.query_start_loc, wl.num_kv_heads, wl.scale, wl.dtype)
    # deep copy: every sequence gets private copies of the shared blocks
    NB = wl.num_blocks
    extra = 3 * wl.num_seqs
    kp = np.concatenate([wl.k_pool, np.zeros((extra,) + wl.k_pool.shape[1:], np.uint16)])
    vp = np.concatenate([wl.v_pool, np.zeros((extra,) + wl.v_pool.shape[1:], np.uint16)])
    tab = wl.block_tables.copy()
    nxt = NB
    for s in range(wl.num_seqs):
        for j in range(3):
            src = wl.block_tables[s, j]
            kp[nxt] = wl.k_pool[src]; vp[nxt] = wl.v_pool[src]
            tab[s, j] = nxt
            nxt += 1
    got, _ = o.attention_ref(wl.q, kp, vp, tab, wl.context_lens, wl.query_start_loc,
                             wl.num_kv_heads, wl.scale, wl.dtype)
    assert np.array_equal(got, base)


def pin_page_block_table_example(o):
    """Tables A = [7,1,3] and B = [7,1,5] from the page: shared blocks 7, 1."""
    with open(os.path.join(GOLDEN, "block_table_example.json")) as f:
        ex = json.load(f)
    nb = ex["pool_blocks"]
    rng = np.random.default_rng(8)
    D, Hkv = 16, 1
    kp = (rng.standard_normal((nb, Hkv, B, D)).astype(np.float16)).view(np.uint16)
    vp = (rng.standard_normal((nb, Hkv, B, D)).astype(np.float16)).view(np.uint16)
    kp[5] = kp[3]; vp[5] = vp[3]          # same content in A's and B's private block
    tables = np.array([ex["table_a"], ex["table_b"]], dtype=np.int32)
    refc = np.bincount(tables.ravel(), minlength=nb)
    assert [int(refc[b]) for b in ex["shared_blocks"]] == [ex["refcount_shared"]] * 2
    q1 = (rng.standard_normal((1, 1, D)).astype(np.float16)).view(np.uint16)
    q = np.concatenate([q1, q1])
    for C in (40, 48):
        ctx = np.array([C, C], np.int32)
        out, _ = o.attention_ref(q, kp, vp, tables, ctx, np.array([0, 1, 2], np.int32), 1,
                                 0.25, "f16")
        assert np.array_equal(out[0], out[1])
        # B's private block changes: only B's output moves
        vp2 = vp.copy(); vp2[5] = (rng.standard_normal((Hkv, B, D)).astype(np.float16)).view(np.uint16)
        out2, _ = o.attention_ref(q, kp, vp2, tables, ctx, np.array([0, 1, 2], np.int32), 1,
                                  0.25, "f16")
        assert np.array_equal(out2[0], out[0]) and not np.array_equal(out2[1], out[1])
        # a shared block changes: both move, identically
        vp3 = vp.copy(); vp3[7] = (rng.standard_normal((Hkv, B, D)).astype(np.float16)).view(np.uint16)
        out3, _ = o.attention_ref(q, kp, vp3, tables, ctx, np.array([0, 1, 2], np.int32), 1,
                                  0.25, "f16")
        assert np.array_equal(out3[0], out3[1]) and not np.array_equal(out3[0], out[0])


def pin_incremental_decode(o):
    """Prefill row i equals a one-row decode over the first C-n+i+1 keys."""
    wl = build_workload("inc", 43, dtype="f16", num_q_heads=4, num_kv_heads=1,
                        cached_lens=[37], new_lens=[21], pool_factor=1.3, new_in_pool=True)
    full, _ = o.attention_ref(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                              wl.query_start_loc, 1, wl.scale, wl.dtype)
    n, C = 21, 58
    for i in range(n):
        one, _ = o.attention_ref(wl.q[i:i + 1], wl.k_pool, wl.v_pool, wl.block_tables,
                                 np.array([C - n + i + 1], np.int32), np.array([0, 1], np.int32),
                                 1, wl.scale, wl.dtype)
        assert np.max(np.abs(one[0] - full[i])) <= 1e-12, i


def pin_chunked_prefill(o):
    """New tokens written and attended in chunks give the one-shot rows."""
    wl = build_workload("chunk", 44, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                        cached_lens=[45], new_lens=[35], pool_factor=1.2)
    kp, vp = o.kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    full, _ = o.attention_ref(wl.q, kp, vp, wl.block_tables, wl.context_lens,
                              wl.query_start_loc, 2, wl.scale, wl.dtype)
    kc, vc = wl.k_pool, wl.v_pool
    for lo, hi in ((0, 9), (9, 10), (10, 27), (27, 35)):
        kc, vc = o.kv_write_ref(kc, vc, wl.k_new[lo:hi], wl.v_new[lo:hi], wl.slot_mapping[lo:hi])
        part, _ = o.attention_ref(wl.q[lo:hi], kc, vc, wl.block_tables,
                                  np.array([45 + hi], np.int32), np.array([0, hi - lo], np.int32),
                                  2, wl.scale, wl.dtype)
        assert np.max(np.abs(part - full[lo:hi])) <= 1e-12, (lo, hi)


def pin_unread_slots_ignored(o):
    """Free blocks, partial-block tails and table padding never reach the output."""
    wl = build_workload("poison", 45, dtype="f16", num_q_heads=4, num_kv_heads=2,
                        cached_lens=[20, 1, 33], new_lens=[5, 1, 2], pool_factor=2.0,
                        extra_table_cols=3)
    kp, vp = o.kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    clean, _ = o.attention_ref(wl.q, kp, vp, wl.block_tables, wl.context_lens,
                               wl.query_start_loc, 2, wl.scale, wl.dtype)
    assert np.all(np.isfinite(clean))
    rng = np.random.default_rng(1)
    kp2, vp2 = kp.copy(), vp.copy()
    refd = np.zeros(wl.num_blocks, bool)
    for s in range(wl.num_seqs):
        nb = -(-int(wl.context_lens[s]) // B)
        refd[wl.block_tables[s, :nb]] = True
    kp2[~refd] = rng.integers(0, 65536, size=kp2[~refd].shape, dtype=np.uint16)
    vp2[~refd] = rng.integers(0, 65536, size=vp2[~refd].shape, dtype=np.uint16)
    tab = wl.block_tables.copy()
    tab[tab < 0] = 1 << 30
    got, _ = o.attention_ref(wl.q, kp2, vp2, tab, wl.context_lens, wl.query_start_loc, 2,
                             wl.scale, wl.dtype)
    assert np.array_equal(got, clean)


# --------------------------------------------------------------------------
# kv_write
# --------------------------------------------------------------------------
def pin_kv_write_slot_arithmetic(o):
    """Slot 37 with 16-token blocks is block 2, offset 5; -1 writes nothing."""
    kp = np.zeros((4, 2, B, 4), np.uint16); vp = np.zeros_like(kp)
    kn = np.arange(2 * 2 * 4, dtype=np.uint16).reshape(2, 2, 4) + 1
    vn = kn + 100
    k2, v2 = o.kv_write_ref(kp, vp, kn, vn, np.array([37, -1], np.int32))
    assert np.array_equal(k2[2, :, 5, :], kn[0]) and np.array_equal(v2[2, :, 5, :], vn[0])
    k2[2, :, 5, :] = 0; v2[2, :, 5, :] = 0
    assert not k2.any() and not v2.any()


def pin_kv_write_round_trip(o):
    """Gathering the written slots returns k_new/v_new bit for bit; nothing else moves."""
    wl = build_workload("rt", 46, dtype="bf16", num_q_heads=2, num_kv_heads=2,
                        cached_lens=[13, 30, 0], new_lens=[20, 2, 17], pool_factor=1.7)
    kp, vp = o.kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    touched = np.zeros(wl.k_pool.shape[0] * B, bool)
    for t, slot in enumerate(wl.slot_mapping):
        b, off = int(slot) // B, int(slot) % B
        assert np.array_equal(kp[b, :, off], wl.k_new[t])
        assert np.array_equal(vp[b, :, off], wl.v_new[t])
        touched[slot] = True
    keep = ~touched.reshape(-1, B)
    for b in range(wl.num_blocks):
        for off in range(B):
            if keep[b, off]:
                assert np.array_equal(kp[b, :, off], wl.k_pool[b, :, off])
                assert np.array_equal(vp[b, :, off], wl.v_pool[b, :, off])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

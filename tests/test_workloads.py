"""Invariants of the seeded input generators (no attention arithmetic here)."""
import math

import numpy as np
import pytest

from workloads import POISON, build_workload, make_config, normal_bits
from workloads.configs import c1, c2, c3, c4, c5

B = 16


def _check_common(wl, pool_factor=None):
    S = wl.num_seqs
    C = wl.context_lens.astype(np.int64)
    n = wl.query_lens
    assert wl.query_start_loc[0] == 0 and wl.query_start_loc[-1] == wl.total_q
    assert np.all(n >= 0) and np.all(n <= C)
    nblk = -(-C // B)
    for s in range(S):
        row = wl.block_tables[s]
        assert np.all(row[:nblk[s]] >= 0) and np.all(row[:nblk[s]] < wl.num_blocks)
        assert np.all(row[nblk[s]:] == -1)
        assert 0 <= nblk[s] * B - C[s] <= B - 1          # fragmentation <= B - 1
    refs = np.concatenate([wl.block_tables[s, :nblk[s]] for s in range(S)])
    assert np.array_equal(np.bincount(refs, minlength=wl.num_blocks), wl.refcounts)
    slots = wl.slot_mapping[wl.slot_mapping >= 0]
    assert np.unique(slots).size == slots.size
    assert np.all(wl.refcounts[slots // B] == 1)          # writes only into private blocks
    if pool_factor is not None:
        need = wl.meta["pool_need"]
        assert wl.num_blocks == math.ceil(pool_factor * need)
    free = wl.refcounts == 0
    assert np.all(wl.k_pool[free] == POISON[wl.dtype])


def test_deterministic_and_thread_independent():
    a = normal_bits(np.random.SeedSequence(5), (3, 1000, 7), "bf16", chunk=1000)
    b = normal_bits(np.random.SeedSequence(5), (3, 1000, 7), "bf16", chunk=1000)
    assert np.array_equal(a, b)
    w1 = build_workload("x", 9, dtype="f16", num_q_heads=4, num_kv_heads=2,
                        cached_lens=[30, 5], new_lens=[2, 5])
    w2 = build_workload("x", 9, dtype="f16", num_q_heads=4, num_kv_heads=2,
                        cached_lens=[30, 5], new_lens=[2, 5])
    for f in ("q", "k_pool", "v_pool", "k_new", "block_tables", "slot_mapping"):
        assert np.array_equal(getattr(w1, f), getattr(w2, f))


def test_bf16_rounding_is_nearest_even():
    from workloads.generate import _round_bits
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-8 + 2**-20], np.float32)
    got = _round_bits(x, "bf16")
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_normal_moments():
    x = normal_bits(np.random.SeedSequence(1), (200000,), "f16").view(np.float16).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_c1_shape():
    wl = c1()
    _check_common(wl)
    assert wl.num_blocks == 64 and wl.context_lens.tolist() == [512]
    assert wl.num_q_heads == wl.num_kv_heads == 8 and wl.dtype == "f16"
    assert sorted(wl.block_tables[0]) == sorted(set(wl.block_tables[0].tolist()))
    assert len(wl.block_tables[0]) == 32


def test_c2_scaled():
    wl = c2(num_seqs=6, lo=128, hi=600, heads=3)
    _check_common(wl, pool_factor=1.2)
    assert wl.max_query_len == 1 and np.all(wl.slot_mapping >= 0)


def test_c3_scaled():
    wl = c3(num_seqs=4, cached_lo=20, cached_hi=90, new_lo=16, new_hi=40, heads=2)
    _check_common(wl, pool_factor=1.2)
    assert np.all(wl.slot_mapping >= 0)


def test_c4_scaled_sharing():
    wl = c4(prompts=3, samples=8, prefix=64, tail_hi=40, q_heads=8, kv_heads=2)
    _check_common(wl, pool_factor=1.2)
    for p in range(3):
        rows = wl.block_tables[p * 8:(p + 1) * 8, :4]
        assert np.all(rows == rows[0])                     # identical prefix entries
        assert np.all(wl.refcounts[rows[0]] == 8)
    tails = wl.context_lens - 64
    assert np.all((wl.slot_mapping == -1) == (tails == 0))


def test_c4_zero_tail_case():
    # a seed where some sample has an empty tail: its newest key is shared, no write
    for seed in range(200):
        wl = c4(seed, prompts=2, samples=4, prefix=32, tail_hi=3, q_heads=4, kv_heads=1)
        if np.any(wl.context_lens == 32):
            break
    _check_common(wl)
    z = np.flatnonzero(wl.context_lens == 32)
    assert z.size and np.all(wl.slot_mapping[z] == -1)


def test_c5_scaled():
    wl = c5(num_seqs=2, cached=64, new=32, q_heads=8, kv_heads=1)
    _check_common(wl, pool_factor=1.1)
    assert wl.context_lens.tolist() == [96, 96]


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c1", "c4", "c5"])
def test_full_configs(name):
    wl = make_config(name)
    _check_common(wl, pool_factor={"c1": None, "c4": 1.2, "c5": 1.1}[name])
    if name == "c5":
        assert wl.num_blocks == 9575 and wl.total_q == 8192
        assert wl.context_lens.tolist() == [34816] * 4

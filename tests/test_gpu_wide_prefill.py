"""The wide prefill kernel (tiles loaded straight into LDS, 256-row
workgroups) vs the CPU oracle, through the C ABI, on an MI355X.

A call goes wide when max_query_len * G >= 1024 (4 waves of 64 rows), and
takes the kernel's 8-wave form (32 rows per wave) when 128 < max_query_len *
G < 1024.  Every (sequence, KV head) pair of such a call, short ones
included, goes through that kernel; the cases below place real rows so that
its edge paths run: a last workgroup whose waves are all, partly or not at
all past the end (in the 8-wave form such waves skip their products), a wave
whose second 32-row half is padding, pairs that fit one 64-key tile,
contexts that end inside a tile (the V rows past the end are cleared),
n == C, empty and decode-only sequences in the same call.
"""
import zlib

import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, run_step, to_dev, wide_rounding_bound
from workloads import build_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()  # fails loudly if the HIP library is not built


# (name, dtype, Hq, Hkv, cached_lens, new_lens); every case has max n*G >= 1024
WIDE = [
    # 1600 rows: 6 full workgroups + one with wave 0 live, waves 1-3 past the end
    ("gqa8_partial_last_wg_bf16", "bf16", 16, 2, [300], [200]),
    # MHA, n == C: 1100 rows, the last workgroup's wave 1 holds 12 real rows
    # in its first half and none in its second
    ("mha_n_equals_c_f16", "f16", 2, 2, [0], [1100]),
    # short pairs (one 64-key tile, 20 rows), decode rows, an empty sequence
    # and a long pair in one wide call
    ("mixed_wide_bf16", "bf16", 8, 2, [0, 700, 50, 9, 2000], [5, 1, 0, 300, 260]),
    ("mixed_wide_f16", "f16", 8, 2, [0, 700, 50, 9, 2000], [5, 1, 0, 300, 260]),
    # contexts ending just past / just before a 64-key tile boundary
    ("tile_edges_bf16", "bf16", 8, 1, [64, 127, 1], [129, 130, 191]),
    # G = 8 with rows exactly filling the workgroups (4 x 256 rows)
    ("exact_fill_f16", "f16", 8, 1, [1000], [128]),
]


# (name, dtype, Hq, Hkv, cached_lens, new_lens); every case has 128 < max n*G < 1024
MID = [
    # 130 rows: waves 0-3 full, wave 4 holds 2 rows, waves 5-7 have none
    ("mid_130_rows_bf16", "bf16", 4, 4, [700, 5], [130, 77]),
    # the multi-turn shape: MHA, runs of 16-256 new tokens over long caches
    ("mid_multiturn_bf16", "bf16", 4, 4, [1024, 3000, 8000, 1500], [16, 256, 129, 200]),
    ("mid_multiturn_f16", "f16", 4, 4, [1024, 3000, 8000, 1500], [16, 256, 129, 200]),
    # 1000 rows (4 items, the last one holds 232 rows), n == C, GQA 4
    ("mid_n_equals_c_f16", "f16", 8, 2, [0, 33], [250, 9]),
    # G = 8, 160 rows; short pairs, decode rows and an empty sequence beside
    ("mid_gqa8_mixed_bf16", "bf16", 8, 1, [0, 300, 64, 17, 900], [20, 1, 0, 7, 12]),
    # contexts ending just past / just before a 64-key tile boundary
    ("mid_tile_edges_f16", "f16", 2, 2, [64, 127, 1], [129, 130, 191]),
    # GQA 2: 300 and 270 rows, whose second items hold 44 and 14 rows (two
    # and one 32-row blocks, each shared by two waves)
    ("mid_small_last_items_bf16", "bf16", 4, 2, [500, 20, 3000], [150, 135, 1]),
]


@pytest.mark.parametrize("case", WIDE + MID, ids=[c[0] for c in WIDE + MID])
def test_wide_cases(case):
    name, dtype, hq, hkv, cached, new = case
    rows = max(new) * (hq // hkv)
    assert rows >= 1024 if case in WIDE else 128 < rows < 1024
    wl = build_workload(name, zlib.crc32(name.encode()) % 10000, dtype=dtype, num_q_heads=hq,
                        num_kv_heads=hkv, cached_lens=cached, new_lens=new, pool_factor=1.3)
    d = to_dev(wl)
    out = run_step(wl, d)
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    err = assert_close(host_bits(out), ref, dtype, what=name)
    print(f"{name}: max|err| = {err:.3e}")


# Calls at the routing boundaries: 128 rows per KV head is the narrow
# kernel's largest call, 129 the 8-wave form's smallest, 1023 its largest and
# 1024 the 4-wave form's smallest.
EDGES = [
    ("narrow_128_rows_bf16", "bf16", 2, 2, [90, 3], [128, 40]),
    ("mid_129_rows_f16", "f16", 2, 2, [90, 3], [129, 40]),
    ("mid_1023_rows_bf16", "bf16", 3, 1, [37, 2], [341, 5]),
    ("wide_1024_rows_f16", "f16", 4, 1, [37, 2], [256, 5]),
]


@pytest.mark.parametrize("case", EDGES, ids=[c[0] for c in EDGES])
def test_routing_boundaries(case):
    name, dtype, hq, hkv, cached, new = case
    wl = build_workload(name, zlib.crc32(name.encode()) % 10000, dtype=dtype, num_q_heads=hq,
                        num_kv_heads=hkv, cached_lens=cached, new_lens=new, pool_factor=1.3)
    d = to_dev(wl)
    out = run_step(wl, d)
    ref, kp, vp = oracle_full(wl)
    err = assert_close(host_bits(out), ref, dtype, what=name)
    print(f"{name}: max|err| = {err:.3e}")


# The same checks for each form: (G, new lengths) giving max n*G >= 1024 or
# 128 < max n*G < 1024.
FORMS = {"wide": (8, [130, 90]), "mid": (2, [130, 90])}


@pytest.mark.parametrize("form", list(FORMS))
def test_unread_slots_never_reach_the_wide_output(form):
    """Free blocks full of random bits (NaN and Inf patterns included) and
    table padding pointing at them leave every output bit unchanged."""
    G, new = FORMS[form]
    args = dict(dtype="bf16", num_q_heads=G, num_kv_heads=1, cached_lens=[150, 33],
                new_lens=new, pool_factor=2.0, extra_table_cols=4)
    wl = build_workload("poison_wide", 21, **args)
    clean = host_bits(run_step(wl, to_dev(wl)))
    free = np.flatnonzero(wl.refcounts == 0)
    assert free.size > 0
    rng = np.random.default_rng(5)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    kp[free] = rng.integers(0, 65536, size=kp[free].shape, dtype=np.uint16)
    vp[free] = rng.integers(0, 65536, size=vp[free].shape, dtype=np.uint16)
    tables = wl.block_tables.copy()
    tables[tables < 0] = free[0]
    wl2 = build_workload("poison_wide", 21, **args)
    wl2.k_pool, wl2.v_pool, wl2.block_tables = kp, vp, tables
    dirty = host_bits(run_step(wl2, to_dev(wl2)))
    assert np.array_equal(clean, dirty)


@pytest.mark.parametrize("form", ["wide", "mid"])
def test_wide_block_permutation_and_repeat_are_bit_identical(form):
    wl = build_workload("perm_wide", 23, dtype="f16", num_q_heads=8 if form == "wide" else 2,
                        num_kv_heads=2, cached_lens=[900, 40], new_lens=[400, 70],
                        pool_factor=1.5)
    d = to_dev(wl)
    base = host_bits(run_step(wl, d))
    again = host_bits(run_step(wl, d, write=False))
    assert np.array_equal(base, again)
    pi = np.random.default_rng(4).permutation(wl.num_blocks)
    kp = np.empty_like(wl.k_pool)
    vp = np.empty_like(wl.v_pool)
    kp[pi] = wl.k_pool
    vp[pi] = wl.v_pool
    tab = np.where(wl.block_tables >= 0, pi[np.maximum(wl.block_tables, 0)], -1)
    slots = np.where(wl.slot_mapping >= 0,
                     pi[np.maximum(wl.slot_mapping, 0) // 16] * 16 + wl.slot_mapping % 16, -1)
    wl.k_pool, wl.v_pool = kp, vp
    wl.block_tables, wl.slot_mapping = tab.astype(np.int32), slots.astype(np.int32)
    got = host_bits(run_step(wl, to_dev(wl)))
    assert np.array_equal(base, got)


@pytest.mark.parametrize("form", ["wide", "mid"])
def test_wide_rescales_when_row_max_grows(form):
    """Keys scaled up along the sequence (key j by 1 + j/40) make every
    row's running max grow by far more than 2^8 in weight again and again,
    so the accumulator rescale runs on every such growth (with N(0,1) keys
    it almost never runs after a row's first keys).  The first sequence's
    items see at least 1024 keys, so they run steady steps (and their
    rescales); the second's see fewer and carry every weight exactly.  The
    weights peak on a few keys here, so the one rounding the wide kernel
    keeps (weights of the steady range rounded to bf16, wide_rounding_bound)
    exceeds 2e-3 + half an ulp: that bound, over exactly those keys, is this
    test's allowance."""
    from oracle import bits_to_f64
    from workloads.generate import _round_bits
    wl = build_workload("grow_wide", 25, dtype="bf16", num_q_heads=8 if form == "wide" else 2,
                        num_kv_heads=2, cached_lens=[1500, 300], new_lens=[300, 260],
                        pool_factor=1.3)
    qsl = wl.query_start_loc
    kp = bits_to_f64(wl.k_pool, wl.dtype)
    kn = bits_to_f64(wl.k_new, wl.dtype)
    seen = set()
    for s in range(wl.num_seqs):
        n = int(qsl[s + 1] - qsl[s])
        cached = int(wl.context_lens[s]) - n
        for j in range(cached):
            b, slot = int(wl.block_tables[s, j // 16]), j % 16
            if (b, slot) not in seen:
                seen.add((b, slot))
                kp[b, :, slot, :] *= 1.0 + j / 40.0
        for i in range(n):
            kn[int(qsl[s]) + i] *= 1.0 + (cached + i) / 40.0
    wl.k_pool = _round_bits(kp.astype(np.float32), wl.dtype)
    wl.k_new = _round_bits(kn.astype(np.float32), wl.dtype)
    d = to_dev(wl)
    out = run_step(wl, d)
    ref, kp_ref, vp_ref = oracle_full(wl)
    err = assert_close(host_bits(out), ref, wl.dtype, what="growing keys",
                       extra=wide_rounding_bound(wl, kp_ref, vp_ref))
    print(f"growing keys: max|err| = {err:.3e}")


@pytest.mark.parametrize("longest", [30, 200], ids=["narrow", "mid"])
def test_more_sequences_than_the_ranking_takes(longest):
    """1100 prefill sequences: past the 1024 that the ranking pass orders,
    sequences keep their given order; every (sequence, head) pair is still
    attended once."""
    rng = np.random.default_rng(401)
    S = 1100
    new = rng.integers(9, 31, size=S)
    new[S // 2] = longest
    cached = rng.integers(0, 100, size=S)
    wl = build_workload(f"many prefill {longest}", 402, dtype="bf16", num_q_heads=2,
                        num_kv_heads=2, cached_lens=cached, new_lens=new, pool_factor=1.2)
    d = to_dev(wl)
    out = run_step(wl, d)
    ref, kp, vp = oracle_full(wl)
    err = assert_close(host_bits(out), ref, "bf16", what=f"{S} sequences")
    print(f"{S} prefill sequences (longest {longest}): max|err| = {err:.3e}")

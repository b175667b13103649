"""HIP path vs the CPU oracle, through the C ABI, on an MI355X.

Every case builds a seeded workload, runs pa_kv_write then pa_attention on
the GPU, and compares with the fp64 oracle: pools bit for bit, attention
outputs within 2e-3.
"""
import zlib

import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, run_step, to_dev
from ws_layout import workspace_layout
from workloads import build_workload, make_config
from workloads.configs import c1, c2, c3, c4, c5

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()  # fails loudly if the HIP library is not built


def _sync():
    import torch
    torch.cuda.synchronize()


# (name, dtype, Hq, Hkv, cached_lens, new_lens)
TINY = [
    ("decode_mha_f16", "f16", 4, 4, [0, 15, 16, 100, 511], [1, 1, 1, 1, 1]),
    ("decode_gqa2_f16", "f16", 8, 4, [33, 700, 5, 1500], [1, 1, 1, 1]),
    ("decode_gqa4_bf16", "bf16", 8, 2, [33, 2047, 5], [1, 1, 1]),
    ("decode_gqa8_f16", "f16", 16, 2, [300, 17], [1, 1]),
    ("decode_g16_to_matrix_cores_bf16", "bf16", 16, 1, [130, 9], [1, 1]),
    ("speculative_rows_f16", "f16", 4, 4, [40, 200, 0], [2, 8, 4]),
    ("prefill_rows9_bf16", "bf16", 3, 1, [70, 0], [3, 9]),
    ("prefill_mha_bf16", "bf16", 2, 2, [0, 40, 100], [16, 24, 130]),
    ("prefill_mha_f16", "f16", 2, 2, [0, 40, 100], [16, 24, 130]),
    ("prefill_gqa8_bf16", "bf16", 16, 2, [200, 13], [40, 70]),
    ("mixed_f16", "f16", 8, 2, [100, 0, 3000, 64], [1, 50, 1, 20]),
    ("empty_sequence_bf16", "bf16", 4, 4, [10, 20, 7], [0, 5, 0]),
    ("long_split_decode_bf16", "bf16", 4, 1, [5000, 100, 2100], [1, 1, 1]),
    ("n_equals_c_f16", "f16", 2, 2, [0], [77]),
    ("single_key_bf16", "bf16", 2, 2, [0, 0], [1, 1]),
]


@pytest.mark.parametrize("case", TINY, ids=[c[0] for c in TINY])
def test_tiny_cases(case):
    name, dtype, hq, hkv, cached, new = case
    wl = build_workload(name, zlib.crc32(name.encode()) % 10000, dtype=dtype, num_q_heads=hq,
                        num_kv_heads=hkv, cached_lens=cached, new_lens=new, pool_factor=1.4)
    d = to_dev(wl)
    out = run_step(wl, d)
    _sync()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    assert np.array_equal(host_bits(d["v_pool"]), vp)
    err = assert_close(host_bits(out), ref, dtype, what=name)
    print(f"{name}: max|err| = {err:.3e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_kv_write_bit_exact(dtype):
    wl = build_workload("kvw", 3, dtype=dtype, num_q_heads=8, num_kv_heads=8,
                        cached_lens=[0, 31, 16, 200], new_lens=[37, 1, 48, 5], pool_factor=2.0)
    # skip every third token: -1 slots must leave the pool alone
    wl.slot_mapping[::3] = -1
    d = to_dev(wl)
    import paged_kv_cache_14_amd as pa
    pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    _sync()
    from oracle import kv_write_ref
    kp, vp = kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    assert np.array_equal(host_bits(d["v_pool"]), vp)


def test_kv_write_many_heads_full_rows():
    # 40 KV heads: a token's K and V rows span 1280 vectors of 16 B
    wl = build_workload("kvw40", 4, dtype="f16", num_q_heads=40, num_kv_heads=40,
                        cached_lens=[3, 50], new_lens=[20, 11], pool_factor=1.5)
    d = to_dev(wl)
    import paged_kv_cache_14_amd as pa
    pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    _sync()
    from oracle import kv_write_ref
    kp, vp = kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    assert np.array_equal(host_bits(d["v_pool"]), vp)


@pytest.mark.parametrize("dtype,hq,hkv,cached,new", [
    ("f16", 4, 4, [77, 300, 16], [1, 1, 1]),          # decode path
    ("bf16", 8, 1, [150, 33], [40, 90]),              # matrix-core path
])
def test_unread_slots_never_reach_the_output(dtype, hq, hkv, cached, new):
    """Free blocks full of random bits (NaN and Inf patterns included) and
    table padding pointing at them leave every output bit unchanged."""
    wl = build_workload("poison", 12, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                        cached_lens=cached, new_lens=new, pool_factor=2.0, extra_table_cols=4)
    d = to_dev(wl)
    clean = host_bits(run_step(wl, d))
    free = np.flatnonzero(wl.refcounts == 0)
    assert free.size > 0
    rng = np.random.default_rng(0)
    kp, vp = wl.k_pool.copy(), wl.v_pool.copy()
    kp[free] = rng.integers(0, 65536, size=kp[free].shape, dtype=np.uint16)
    vp[free] = rng.integers(0, 65536, size=vp[free].shape, dtype=np.uint16)
    tables = wl.block_tables.copy()
    tables[tables < 0] = free[0]  # in range, so a stray read lands in garbage, not a fault
    wl2 = build_workload("poison", 12, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                         cached_lens=cached, new_lens=new, pool_factor=2.0, extra_table_cols=4)
    wl2.k_pool, wl2.v_pool, wl2.block_tables = kp, vp, tables
    dirty = host_bits(run_step(wl2, to_dev(wl2)))
    assert np.array_equal(clean, dirty)


@pytest.mark.parametrize("dtype,hq,hkv,cached,new", [
    ("f16", 8, 8, [500, 47], [1, 1]),
    ("bf16", 8, 2, [260, 31], [50, 20]),
])
def test_block_permutation_is_bit_identical(dtype, hq, hkv, cached, new):
    wl = build_workload("perm", 13, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                        cached_lens=cached, new_lens=new, pool_factor=1.5)
    base = host_bits(run_step(wl, to_dev(wl)))
    pi = np.random.default_rng(2).permutation(wl.num_blocks)
    kp = np.empty_like(wl.k_pool); vp = np.empty_like(wl.v_pool)
    kp[pi] = wl.k_pool; vp[pi] = wl.v_pool
    tab = np.where(wl.block_tables >= 0, pi[np.maximum(wl.block_tables, 0)], -1)
    slots = np.where(wl.slot_mapping >= 0,
                     pi[np.maximum(wl.slot_mapping, 0) // 16] * 16 + wl.slot_mapping % 16, -1)
    wl.k_pool, wl.v_pool = kp, vp
    wl.block_tables, wl.slot_mapping = tab.astype(np.int32), slots.astype(np.int32)
    got = host_bits(run_step(wl, to_dev(wl)))
    assert np.array_equal(base, got)


def _privatise(wl, blocks):
    """Copy the first `blocks` table entries of every sequence to private blocks."""
    NB = wl.num_blocks
    copies = []
    tab = wl.block_tables.copy()
    for s in range(wl.num_seqs):
        for j in range(blocks):
            copies.append(tab[s, j])
            tab[s, j] = NB + len(copies) - 1
    wl.k_pool = np.concatenate([wl.k_pool, wl.k_pool[copies]])
    wl.v_pool = np.concatenate([wl.v_pool, wl.v_pool[copies]])
    wl.block_tables = tab


def test_shared_prefix_matches_private_copies():
    """Samples sharing prefix blocks (refcount 8) and the same data laid out
    privately both match the oracle.  Shared prefixes of 4 blocks or more go
    through the matrix cores once per group, so only the order of the fp32
    sums separates the two layouts."""
    wl = c4(9, prompts=2, samples=8, prefix=256, tail_hi=40, q_heads=8, kv_heads=2)
    ref, kp, vp = oracle_full(wl)
    shared = host_bits(run_step(wl, to_dev(wl)))
    assert_close(shared, ref, "bf16", what="shared prefix")
    _privatise(wl, 256 // 16)
    private = host_bits(run_step(wl, to_dev(wl)))
    assert_close(private, ref, "bf16", what="private copies")


def test_short_shared_prefix_is_bit_identical_to_private_copies():
    """A prefix of 3 shared blocks is below the grouping threshold: the plain
    decode path reads it per sample, bit for bit as from private copies."""
    wl = c4(10, prompts=2, samples=8, prefix=48, tail_hi=40, q_heads=8, kv_heads=2)
    shared = host_bits(run_step(wl, to_dev(wl)))
    _privatise(wl, 48 // 16)
    private = host_bits(run_step(wl, to_dev(wl)))
    assert np.array_equal(shared, private)


def test_side_stream_and_repeat_calls():
    import torch
    wl = build_workload("stream", 14, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                        cached_lens=[600, 90], new_lens=[1, 30], pool_factor=1.3)
    d = to_dev(wl)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = host_bits(run_step(wl, d, stream=s))
    b = host_bits(run_step(wl, d, write=False))
    assert np.array_equal(a, b)


SCALED = {
    "c1": lambda: c1(),
    "c2": lambda: c2(num_seqs=8, lo=128, hi=1500, heads=8),
    "c3": lambda: c3(num_seqs=4, cached_lo=1024, cached_hi=1600, new_lo=16, new_hi=256, heads=4),
    "c4": lambda: c4(prompts=2, samples=8, prefix=2048, tail_hi=512, q_heads=32, kv_heads=8),
    "c5": lambda: c5(num_seqs=1, cached=4096, new=512, q_heads=64, kv_heads=8),
}


@pytest.mark.parametrize("name", sorted(SCALED))
def test_config_scaled_full_compare(name):
    """Each workload's structure at a size the oracle finishes in seconds; every output."""
    wl = SCALED[name]()
    d = to_dev(wl)
    out = run_step(wl, d)
    _sync()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    err = assert_close(host_bits(out), ref, wl.dtype, bare=True, what=name)
    print(f"{name} scaled: max|err| = {err:.3e}")


def _samples(wl, count, seed):
    rng = np.random.default_rng(seed)
    Tq, Hq = wl.total_q, wl.num_q_heads
    picks = {(int(t), int(h)) for t, h in zip(rng.integers(0, Tq, count), rng.integers(0, Hq, count))}
    qsl = wl.query_start_loc
    for s in range(wl.num_seqs):      # first and last row of every sequence, head 0 and last
        if qsl[s + 1] > qsl[s]:
            for t in (int(qsl[s]), int(qsl[s + 1]) - 1):
                picks.add((t, 0))
                picks.add((t, Hq - 1))
    return sorted(picks)


def _full_size_step(name):
    """A full-size workload through kv_write + attention, in the bench's launch
    configuration; returns the workload, the output bits and the oracle's pools
    (checked bit for bit against the GPU's)."""
    from oracle import bits_to_f64, kv_write_ref
    wl = make_config(name)
    print(f"[full size] {name}: {wl.num_seqs} sequences, {wl.total_q} query tokens", flush=True)
    d = to_dev(wl)
    out = run_step(wl, d)
    _sync()
    got = host_bits(out)
    assert np.all(np.isfinite(bits_to_f64(got, wl.dtype)))
    kp, vp = kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    assert np.array_equal(host_bits(d["v_pool"]), vp)
    return wl, got, kp, vp


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_config_full_size_every_output(name):
    """Full-size workloads in the bench's launch configuration, every output
    against the fp64 oracle at the bare 2e-3."""
    from oracle import attention_ref
    wl, got, kp, vp = _full_size_step(name)
    ref, _ = attention_ref(wl.q, kp, vp, wl.block_tables, wl.context_lens, wl.query_start_loc,
                           wl.num_kv_heads, wl.scale, wl.dtype)
    err = assert_close(got, ref, wl.dtype, bare=True, what=f"{name} full size, every output")
    print(f"{name} full size: max|err| = {err:.3e}")


def test_config_c5_full_size_sampled():
    """The long-context chunked prefill at full size (9 TFLOP: minutes of fp64
    on the host), checked on sampled outputs, first and last row of every
    sequence included; its structure is compared on every output below."""
    from oracle import attention_ref_sample
    wl, got, kp, vp = _full_size_step("c5")
    picks = _samples(wl, 160, 17)
    ref = attention_ref_sample(wl.q, kp, vp, wl.block_tables, wl.context_lens,
                               wl.query_start_loc, wl.num_kv_heads, wl.scale, wl.dtype, picks)
    sel = np.stack([got[t, h] for t, h in picks])
    err = assert_close(sel, ref, wl.dtype, bare=True, what=f"c5 full ({len(picks)} sampled rows)")
    print(f"c5 full ({len(picks)} sampled rows): max|err| = {err:.3e}")


def test_c5_shape_more_items_than_workgroups():
    """Chunked prefill, GQA 64/8, 2 x (4096 cached + 2048 new): 16 (sequence,
    KV head) pairs of 64 256-row items each, 1024 items for the 256 persistent
    workgroups, so every workgroup carries state from item to item.  Every
    output against the oracle at the bare 2e-3."""
    wl = c5(seed=5, num_seqs=2, cached=4096, new=2048, q_heads=64, kv_heads=8)
    print(f"[c5 shape] {wl.num_seqs} x ({4096} + {2048}), 64/8 heads", flush=True)
    d = to_dev(wl)
    out = run_step(wl, d)
    _sync()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    err = assert_close(host_bits(out), ref, wl.dtype, bare=True, what="c5 shape, 1024 items")
    print(f"c5 shape, 1024 items: max|err| = {err:.3e}")


def test_workspace_reused_across_calls_and_data():
    """One workspace, calls on different data back to back: every call is right.

    The decode merge passes partial results between workgroups through the
    workspace; a stale record from an earlier call must never be merged.
    """
    import torch
    import paged_kv_cache_14_amd as pa
    wls = [build_workload("ws", seed, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                          cached_lens=[3000, 1500, 700, 20], new_lens=[1, 1, 1, 1],
                          pool_factor=1.2) for seed in (31, 32)]
    refs = [oracle_full(wl)[0] for wl in wls]
    devs = [to_dev(wl) for wl in wls]
    for wl, d in zip(wls, devs):
        pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    wl0 = wls[0]
    need = pa.pa_attention_workspace_size(wl0.num_seqs, wl0.total_q, 8, 2, 128, 3001, 1)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    firsts = {}
    for rep in range(6):
        i = rep % 2
        wl, d = wls[i], devs[i]
        out = pa.pa_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"],
                              d["context_lens"], d["query_start_loc"], 2, wl.scale,
                              max_query_len=1, max_context_len=3001, workspace=ws)
        got = host_bits(out)
        assert_close(got, refs[i], "bf16", what=f"call {rep}")
        if i in firsts:
            assert np.array_equal(got, firsts[i])
        firsts[i] = got
        # the decode's ticket counters are back at zero after every call
        lay = workspace_layout(wl0.num_seqs, 8, 2, 3001, 1)
        assert lay["total"] == need
        assert lay["counters_bytes"] > 0 and lay["counters"] == 256
        zero = ws[:lay["zero_bytes"]]
        assert int(zero.view(torch.int32).abs().sum().item()) == 0, f"call {rep}"

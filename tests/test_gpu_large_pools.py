"""Pools whose byte offsets pass 2^31 and 2^32: every kernel forms K/V
addresses in 64 bits.

An MI355X holds 288 GB, so a serving pool of many GiB is the ordinary case,
and a block id times the block's bytes overflows 32 bits from about 4 GiB on
(2 GiB where the product is signed).  Each case builds a batch in a compact
pool, then places that pool's blocks at the top of a device pool of more than
4.5 GiB per K and per V (block ids shifted, slots shifted by the same number
of blocks), with the memory below it zeroed.  pa_kv_write then pa_attention
run on the large pools, and the results must match the oracle on the compact
batch: the written blocks bit for bit, every output within 2e-3 plus half an
output ulp, and not one byte below the placed blocks changed.  The routes
covered: the decode on the vector ALUs with split-K merges, the matrix-core
decode with the shared-prefix plan and pass, the narrow prefill, both forms
of the wide prefill, pa_copy_blocks between high block ids, the
quantization of pages from high blocks with the decode over them, and swaps
between high blocks and a pinned host tier (by kernel and through staging).
"""
import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, torch_dtype
from workloads import build_workload

pytestmark = pytest.mark.gpu

LOW_BYTES = 9 << 29  # 4.5 GiB of pool below the placed blocks


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()  # fails loudly if the HIP library is not built


def _place_high(wl):
    """Device tensors of the batch with its pool placed above LOW_BYTES in
    zeroed pools; returns (tensors, block offset)."""
    import torch
    import paged_kv_cache_14_amd as pa
    tdt = torch_dtype(wl.dtype)
    nb, hkv, bs, d = wl.k_pool.shape
    block_bytes = hkv * bs * d * 2
    off = -(-LOW_BYTES // block_bytes)
    assert off * block_bytes > (1 << 32)
    bt = np.where(wl.block_tables >= 0, wl.block_tables + off, wl.block_tables).astype(np.int32)
    sm = np.where(wl.slot_mapping >= 0, wl.slot_mapping + off * bs, wl.slot_mapping).astype(np.int32)
    pa.pa_check_batch(bt, wl.context_lens, wl.query_start_loc, off + nb, sm,
                      slots_are_new_tokens=True)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to("cuda:0")

    def d32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")

    k_pool = torch.zeros((off + nb, hkv, bs, d), dtype=tdt, device="cuda:0")
    v_pool = torch.zeros_like(k_pool)
    k_pool[off:] = d16(wl.k_pool)
    v_pool[off:] = d16(wl.v_pool)
    return dict(q=d16(wl.q), k_pool=k_pool, v_pool=v_pool, k_new=d16(wl.k_new),
                v_new=d16(wl.v_new), slot_mapping=d32(sm), block_tables=d32(bt),
                context_lens=d32(wl.context_lens),
                query_start_loc=d32(wl.query_start_loc)), off


def _low_region_untouched(d, off):
    import torch
    for name in ("k_pool", "v_pool"):
        low = d[name][:off].view(torch.int16)
        assert int(torch.count_nonzero(low)) == 0, f"a write landed below the placed {name} blocks"


CASES = [
    # (name, dtype, Hq, Hkv, cached, new, shared-prefix group)
    ("valu_decode_split_f16", "f16", 8, 8, [20000, 5, 700, 3000], [1, 1, 1, 1], None),
    ("mfma_decode_shared_prefix_bf16", "bf16", 32, 8, [900, 40], [1, 1], (5, 20)),
    ("narrow_prefill_bf16", "bf16", 16, 4, [1500, 0, 300], [30, 17, 1], None),
    ("wide_8wave_bf16", "bf16", 16, 4, [1200, 64, 5], [100, 60, 1], None),
    ("wide_4wave_f16", "f16", 16, 2, [2100, 30], [200, 1], None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pool_beyond_4_gib(case):
    import torch
    import paged_kv_cache_14_amd as pa
    name, dtype, hq, hkv, cached, new, group = case
    cached, new, groups, prefix_blocks = list(cached), list(new), None, 0
    if group is not None:
        members, prefix_blocks = group
        first = len(cached)
        cached += [prefix_blocks * 16 + 37 * i for i in range(members)]
        new += [1] * members
        groups = [list(range(first, first + members))]
    wl = build_workload(name, 500 + len(name), dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                        cached_lens=cached, new_lens=new, pool_factor=1.2,
                        shared_prefix_groups=groups, shared_prefix_blocks=prefix_blocks)
    print(f"{name}: placing {wl.num_blocks} blocks above {LOW_BYTES / 2**30:.1f} GiB", flush=True)
    d, off = _place_high(wl)
    pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    out = pa.pa_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                          d["query_start_loc"], wl.num_kv_heads, wl.scale,
                          max_query_len=wl.max_query_len, max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"][off:]), kp)
    assert np.array_equal(host_bits(d["v_pool"][off:]), vp)
    err = assert_close(host_bits(out), ref, wl.dtype, what=name)
    _low_region_untouched(d, off)
    print(f"{name}: block ids from {off}, max|err| = {err:.3e}")
    if name.startswith("valu"):
        # copy-on-write copies between high block ids, bit for bit
        rng = np.random.default_rng(77)
        src = rng.choice(wl.num_blocks, size=6, replace=False)
        dst = np.setdiff1d(np.arange(wl.num_blocks), src)[rng.permutation(wl.num_blocks - 6)[:6]]
        pa.pa_copy_blocks(d["k_pool"], d["v_pool"],
                          torch.from_numpy((src + off).astype(np.int32)).to("cuda:0"),
                          torch.from_numpy((dst + off).astype(np.int32)).to("cuda:0"))
        torch.cuda.synchronize()
        kp[dst], vp[dst] = kp[src], vp[src]
        assert np.array_equal(host_bits(d["k_pool"][off:]), kp)
        assert np.array_equal(host_bits(d["v_pool"][off:]), vp)
        _low_region_untouched(d, off)
    del d, out
    torch.cuda.empty_cache()


def test_quantized_pages_from_blocks_beyond_4_gib():
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import kv_write_ref
    from oracle.quant_ref import attention_quant_ref
    from test_gpu_quant import PAGE_BYTES, _same_page, oracle_pages, quant_setup, unpack_page
    wl = build_workload("quant high", 530, dtype="bf16", num_q_heads=16, num_kv_heads=4,
                        cached_lens=[3000, 129, 700, 2047], new_lens=[1, 1, 1, 1],
                        pool_factor=1.2)
    d, off = _place_high(wl)

    def d32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")

    pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    quant, page_tables, src, npages = quant_setup(wl)
    qpool = torch.zeros((npages, wl.num_kv_heads, PAGE_BYTES), dtype=torch.uint8, device="cuda:0")
    pa.pa_quantize_pages(qpool, d["k_pool"], d["v_pool"],
                         d32(np.arange(npages, dtype=np.int32)), d32(src + off))
    out = pa.pa_attention_quant(d["q"], qpool, d32(page_tables), d32(quant), d["k_pool"],
                                d["v_pool"], d["block_tables"], d["context_lens"],
                                d["query_start_loc"], wl.num_kv_heads, wl.scale,
                                max_query_len=wl.max_query_len,
                                max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    kp, vp = kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    pages = oracle_pages(wl, kp, vp, quant, page_tables)
    got_pool = qpool.cpu().numpy()
    for s in range(wl.num_seqs):  # every page, bit for bit
        for p in range(int(quant[s]) // 128):
            for g in range(wl.num_kv_heads):
                _same_page(unpack_page(got_pool[page_tables[s, p], g]), pages[s][g][p],
                           f"seq {s} page {p} head {g}")
    ref = attention_quant_ref(wl.q, pages, kp, vp, wl.block_tables, wl.context_lens, quant,
                              wl.query_start_loc, wl.num_kv_heads, wl.scale, wl.dtype)
    err = assert_close(host_bits(out), ref, wl.dtype, what="quantized pages from high blocks")
    _low_region_untouched(d, off)
    print(f"quantized pages from block ids {off}+: {npages} pages, max|err| = {err:.3e}")
    del d, out, qpool
    torch.cuda.empty_cache()


def test_swaps_with_blocks_beyond_4_gib():
    """Swap-out from high device blocks to a pinned host tier and swap-in back
    to other high blocks, by the copy kernel and through a staging run: bit
    for bit, nothing below the high blocks touched."""
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import swap_blocks_ref
    rng = np.random.default_rng(531)
    H, B, D, NG, NH = 8, 16, 128, 120, 100
    off = -(-LOW_BYTES // (H * B * D * 2))
    tdt = torch_dtype("bf16")
    gk = rng.integers(0, 65536, size=(NG, H, B, D), dtype=np.uint16)
    gv = rng.integers(0, 65536, size=(NG, H, B, D), dtype=np.uint16)

    def dev(a):
        return torch.from_numpy(a.view(np.int16)).view(tdt).to("cuda:0")

    def d32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")

    k = torch.zeros((off + NG, H, B, D), dtype=tdt, device="cuda:0")
    v = torch.zeros_like(k)
    k[off:], v[off:] = dev(gk), dev(gv)
    d = dict(k_pool=k, v_pool=v)
    hk0 = rng.integers(0, 65536, size=(NH, H, B, D), dtype=np.uint16)
    hv0 = rng.integers(0, 65536, size=(NH, H, B, D), dtype=np.uint16)
    hk = torch.from_numpy(hk0.view(np.int16)).view(tdt).pin_memory()
    hv = torch.from_numpy(hv0.view(np.int16)).view(tdt).pin_memory()
    out_src, out_dst = rng.permutation(NG)[:50], rng.permutation(NH)[:50]
    pa.pa_swap_blocks(hk, hv, k, v, d32(out_src + off), d32(out_dst))      # swap-out
    torch.cuda.synchronize()
    hk1, hv1 = swap_blocks_ref(hk0, hv0, gk, gv, out_src, out_dst)
    assert np.array_equal(hk.view(torch.int16).numpy().view(np.uint16), hk1)
    assert np.array_equal(hv.view(torch.int16).numpy().view(np.uint16), hv1)
    back = rng.permutation(NG)[:50]
    pa.pa_swap_blocks(k, v, hk, hv, d32(out_dst), d32(back + off))         # swap-in
    torch.cuda.synchronize()
    gk2, gv2 = swap_blocks_ref(gk, gv, hk1, hv1, out_dst, back)
    assert np.array_equal(host_bits(k[off:]), gk2) and np.array_equal(host_bits(v[off:]), gv2)
    # the same through a staging run and a contiguous host run
    ids = rng.permutation(NG)[:40]
    rk = torch.empty((40, H, B, D), dtype=tdt).pin_memory()
    rv = torch.empty((40, H, B, D), dtype=tdt).pin_memory()
    sk = torch.empty((48, H, B, D), dtype=tdt, device="cuda:0")
    sv = torch.empty((48, H, B, D), dtype=tdt, device="cuda:0")
    pa.pa_swap_out_staged(rk, rv, k, v, sk, sv, d32(ids + off))
    torch.cuda.synchronize()
    assert np.array_equal(rk.view(torch.int16).numpy().view(np.uint16), gk2[ids])
    assert np.array_equal(rv.view(torch.int16).numpy().view(np.uint16), gv2[ids])
    back2 = rng.permutation(NG)[:40]
    pa.pa_swap_in_staged(k, v, rk, rv, sk, sv, d32(back2 + off))
    torch.cuda.synchronize()
    gk3, gv3 = swap_blocks_ref(gk2, gv2, gk2[ids], gv2[ids], np.arange(40), back2)
    assert np.array_equal(host_bits(k[off:]), gk3) and np.array_equal(host_bits(v[off:]), gv3)
    _low_region_untouched(d, off)
    del d, k, v, sk, sv
    torch.cuda.empty_cache()

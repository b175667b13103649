"""Block management on an MI355X: pa_copy_blocks bit for bit against the
oracle's copy, and whole steps driven by libpa's host block manager (forks,
prefix shares, copy-on-write, the shared-prefix GQA decode workload built
through it) against the oracle's block-management model and attention.

The GPU side runs: manager -> pa_copy_blocks -> pa_kv_write -> pa_attention.
The oracle side runs: model -> copy_blocks_ref -> kv_write_ref ->
attention_ref.  The two managers must agree on every slot, copy and table
(checked on the way); pools must agree bit for bit; outputs within 2e-3.
"""
import numpy as np
import pytest

from gpu_util import assert_close, host_bits, torch_dtype
from workloads import normal_bits

pytestmark = pytest.mark.gpu
B = 16
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()


def _d16(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch_dtype(dtype)).cuda()


def _d32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype,heads", [("f16", 1), ("bf16", 8), ("f16", 40)])
def test_copy_blocks_bit_exact(dtype, heads):
    """Random bit patterns (NaN and Inf included) in every block; a list of
    copies into distinct fresh blocks; blocks outside the list untouched."""
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import copy_blocks_ref
    rng = np.random.default_rng(heads)
    NB = 300
    kp = rng.integers(0, 65536, size=(NB, heads, B, D), dtype=np.uint16)
    vp = rng.integers(0, 65536, size=(NB, heads, B, D), dtype=np.uint16)
    perm = rng.permutation(NB)
    src, dst = perm[:70], perm[70:140]
    k, v = _d16(kp, dtype), _d16(vp, dtype)
    pa.pa_copy_blocks(k, v, _d32(src), _d32(dst))
    torch.cuda.synchronize()
    kw, vw = copy_blocks_ref(kp, vp, src, dst)
    assert np.array_equal(host_bits(k), kw)
    assert np.array_equal(host_bits(v), vw)


def test_copy_blocks_ids_out_of_range_are_skipped():
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import copy_blocks_ref
    rng = np.random.default_rng(5)
    kp = rng.integers(0, 65536, size=(16, 2, B, D), dtype=np.uint16)
    vp = rng.integers(0, 65536, size=(16, 2, B, D), dtype=np.uint16)
    k, v = _d16(kp, "bf16"), _d16(vp, "bf16")
    pa.pa_copy_blocks(k, v, _d32([3, 16, -1, 5]), _d32([9, 2, 4, 99]))
    torch.cuda.synchronize()
    kw, vw = copy_blocks_ref(kp, vp, [3], [9])
    assert np.array_equal(host_bits(k), kw) and np.array_equal(host_bits(v), vw)


class Program:
    """Runs block-management operations on libpa's manager and on the
    oracle's model side by side, checking that they agree, and records what
    the GPU and the oracle must each do with the pools."""

    def __init__(self, num_blocks, num_kv_heads, dtype, seed, free_order=None):
        import paged_kv_cache_14_amd as pa
        from oracle import BlockManagerRef
        order = free_order if free_order is not None else \
            np.random.default_rng(seed).permutation(num_blocks)
        self.bm = pa.BlockManager(num_blocks, order)
        self.ref = BlockManagerRef(num_blocks, order)
        self.NB, self.Hkv, self.dtype, self.seed = num_blocks, num_kv_heads, dtype, seed
        self.steps = []   # ("copy", src, dst) and ("write", slots, k_new, v_new), in order
        self.n_writes = 0

    def add(self):
        a, b = self.bm.add_sequence(), self.ref.add_sequence()
        assert a == b
        return a

    def fork(self, p):
        a, b = self.bm.fork(p), self.ref.fork(p)
        assert a == b
        return a

    def share(self, p, n):
        a, b = self.bm.share_prefix(p, n), self.ref.share_prefix(p, n)
        assert a == b
        return a

    def free(self, s):
        self.bm.free_sequence(s)
        self.ref.free_sequence(s)

    def append(self, s, n):
        slots, copies = self.bm.append(s, n)
        want_slots, want_copies = self.ref.append(s, n)
        assert list(slots) == want_slots and copies == want_copies
        for src, dst in copies:
            self.steps.append(("copy", [src], [dst]))
        ss = np.random.SeedSequence([self.seed, 7, self.n_writes])
        ka, kb = ss.spawn(2)
        self.n_writes += 1
        self.steps.append(("write", np.asarray(want_slots, np.int32),
                           normal_bits(ka, (n, self.Hkv, D), self.dtype),
                           normal_bits(kb, (n, self.Hkv, D), self.dtype)))
        return copies

    def tables(self, seqs):
        width = max(1, max(len(self.ref.table(s)) for s in seqs))
        tab, lens = self.bm.tables(seqs, width)
        want, want_lens = self.ref.tables_array(seqs, width)
        assert np.array_equal(tab, want) and np.array_equal(lens, want_lens)
        return want, want_lens

    def pools(self):
        """(GPU pools after the steps, oracle pools after the same steps).
        Consecutive writes go as one kv_write while their slots stay distinct;
        a copy first flushes the writes before it."""
        import torch
        import paged_kv_cache_14_amd as pa
        from oracle import copy_blocks_ref, kv_write_ref
        nan = np.uint16(0x7E00)
        kp = np.full((self.NB, self.Hkv, B, D), nan, np.uint16)
        vp = kp.copy()
        k, v = _d16(kp, self.dtype), _d16(vp, self.dtype)
        pending = []

        def flush():
            nonlocal kp, vp
            if not pending:
                return
            slots = np.concatenate([w[0] for w in pending])
            kn = np.concatenate([w[1] for w in pending])
            vn = np.concatenate([w[2] for w in pending])
            pending.clear()
            pa.pa_check_batch(np.zeros((0, 1), np.int32), np.zeros(0, np.int32),
                              np.zeros(1, np.int32), self.NB, slots)
            pa.pa_kv_write(_d16(kn, self.dtype), _d16(vn, self.dtype), k, v, _d32(slots))
            kp, vp = kv_write_ref(kp, vp, kn, vn, slots)

        seen = set()
        for st in self.steps:
            if st[0] == "copy":
                flush()
                seen.clear()
                pa.pa_copy_blocks(k, v, _d32(st[1]), _d32(st[2]))
                kp, vp = copy_blocks_ref(kp, vp, st[1], st[2])
            else:
                _, slots, kn, vn = st
                if seen & set(slots.tolist()):
                    flush()
                    seen.clear()
                seen.update(slots.tolist())
                pending.append((slots, kn, vn))
        flush()
        torch.cuda.synchronize()
        return k, v, kp, vp


def _decode_step(prog, seqs, num_q_heads, what):
    """One decode token per sequence (its newest key is the last it sees)."""
    import paged_kv_cache_14_amd as pa
    from oracle import attention_ref
    k, v, kp, vp = prog.pools()
    assert np.array_equal(host_bits(k), kp), f"{what}: K pool"
    assert np.array_equal(host_bits(v), vp), f"{what}: V pool"
    tab, lens = prog.tables(seqs)
    S = len(seqs)
    q = normal_bits(np.random.SeedSequence([prog.seed, 99]), (S, num_q_heads, D), prog.dtype)
    qsl = np.arange(S + 1, dtype=np.int32)
    pa.pa_check_batch(tab, lens, qsl, prog.NB)
    out = pa.pa_attention(_d16(q, prog.dtype), k, v, _d32(tab), _d32(lens), _d32(qsl),
                          prog.Hkv, D ** -0.5, max_query_len=1, max_context_len=int(lens.max()))
    ref, _ = attention_ref(q, kp, vp, tab, lens, qsl, prog.Hkv, D ** -0.5, prog.dtype)
    return assert_close(host_bits(out), ref, prog.dtype, what=what)


def test_fork_and_prefix_share_with_copy_on_write():
    """A prompt of 40 tokens (its last block partly filled) forked three ways
    and shared as a 20-token prefix; each sequence then appends.  The first
    writers into the shared last block copy it; the last one writes in place."""
    prog = Program(40, 2, "bf16", 31)
    a = prog.add()
    prog.append(a, 40)
    kids = [prog.fork(a) for _ in range(3)]
    d = prog.share(a, 20)
    n_copies = 0
    for s in kids + [a]:
        n_copies += len(prog.append(s, 5))
    n_copies += len(prog.append(d, 30))
    assert n_copies == 4  # three of the four 40-token sequences, and the prefix
    assert prog.ref.refcount[prog.ref.table(a)[0]] == 5   # block 0: all five sequences
    _decode_step(prog, kids + [a, d], 8, "fork + prefix share + CoW")


def test_shared_prefix_decode_built_through_the_manager():
    """The GQA shared-prefix decode shape, scaled down, built by the manager:
    per prompt, one sequence appends a 250-token prefix (last block partly
    filled) and is forked into 8 samples, each appending its own tail; the
    prompt's first 15 blocks end with reference count 8, the partly filled
    16th is copied by 7 of the 8 samples.  The decode batch then takes the
    shared-prefix path (groups of 8)."""
    rng = np.random.default_rng(44)
    prompts, samples, prefix, hq, hkv = 4, 8, 250, 16, 4
    need = prompts * (16 + samples * 8)
    prog = Program(int(need * 1.2), hkv, "bf16", 45)
    seqs = []
    for _ in range(prompts):
        base = prog.add()
        prog.append(base, prefix)
        kids = [prog.fork(base) for _ in range(samples)]
        prog.free(base)
        first = prog.ref.table(kids[0])
        assert all(prog.ref.refcount[blk] == samples for blk in first)
        copies = sum(len(prog.append(s, int(rng.integers(1, 100)))) for s in kids)
        assert copies == samples - 1
        assert all(prog.ref.refcount[blk] == samples for blk in first[:15])
        seqs += kids
    _decode_step(prog, seqs, hq, "shared-prefix decode through the manager")


def test_full_size_shared_prefix_decode_built_through_the_manager():
    """The full GQA shared-prefix decode: 32 prompts x 8 samples, a 2048-token
    prefix (128 blocks, reference count 8) and tails of U[0, 512] tokens,
    32/8 heads, bf16, from a shuffled free list 1.2x the unique need; every
    output against the oracle."""
    rng = np.random.default_rng(4)
    prompts, samples, prefix, hq, hkv = 32, 8, 2048, 32, 8
    tails = rng.integers(0, 512, size=(prompts, samples), endpoint=True)
    need = prompts * prefix // B + int(np.sum(-(-tails // B)))
    prog = Program(int(np.ceil(1.2 * need)), hkv, "bf16", 46)
    seqs = []
    for p in range(prompts):
        base = prog.add()
        prog.append(base, prefix)
        kids = [prog.fork(base) for _ in range(samples)]
        prog.free(base)
        for s, t in zip(kids, tails[p]):
            assert prog.append(s, int(t)) == []   # 2048 fills whole blocks: no copy
        assert all(prog.ref.refcount[blk] == samples for blk in prog.ref.table(kids[0])[:128])
        seqs += kids
    print(f"[blocks] full-size shared-prefix decode: {len(seqs)} sequences, "
          f"{prog.NB} blocks", flush=True)
    err = _decode_step(prog, seqs, hq, "full-size shared-prefix decode through the manager")
    print(f"full-size through the manager: max|err| = {err:.3e}")


@pytest.mark.parametrize("dtype,heads", [("bf16", 8), ("f16", 40)])
def test_swap_round_trip_through_a_pinned_host_tier(dtype, heads):
    """GPU blocks swapped out to a pinned host tier, then back in under other
    ids: both transfers bit for bit against the oracle's copy, everything
    outside the lists untouched; a pageable host pool is refused."""
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import swap_blocks_ref
    rng = np.random.default_rng(heads + 100)
    NG, NH = 200, 300
    gk = rng.integers(0, 65536, size=(NG, heads, B, D), dtype=np.uint16)
    gv = rng.integers(0, 65536, size=(NG, heads, B, D), dtype=np.uint16)
    hk0 = rng.integers(0, 65536, size=(NH, heads, B, D), dtype=np.uint16)
    hv0 = rng.integers(0, 65536, size=(NH, heads, B, D), dtype=np.uint16)
    tdt = torch_dtype(dtype)
    k, v = _d16(gk, dtype), _d16(gv, dtype)
    hk = torch.from_numpy(hk0.view(np.int16)).view(tdt).pin_memory()
    hv = torch.from_numpy(hv0.view(np.int16)).view(tdt).pin_memory()
    out_src = rng.permutation(NG)[:90]
    out_dst = rng.permutation(NH)[:90]
    pa.pa_swap_blocks(hk, hv, k, v, _d32(out_src), _d32(out_dst))   # swap-out
    torch.cuda.synchronize()
    hk1, hv1 = swap_blocks_ref(hk0, hv0, gk, gv, out_src, out_dst)
    assert np.array_equal(hk.view(torch.int16).numpy().view(np.uint16), hk1)
    assert np.array_equal(hv.view(torch.int16).numpy().view(np.uint16), hv1)
    back = rng.permutation(NG)[:90]
    pa.pa_swap_blocks(k, v, hk, hv, _d32(out_dst), _d32(back))      # swap-in, other ids
    torch.cuda.synchronize()
    gk2, gv2 = swap_blocks_ref(gk, gv, hk1, hv1, out_dst, back)
    assert np.array_equal(host_bits(k), gk2) and np.array_equal(host_bits(v), gv2)
    for s, d in zip(out_src, back):
        assert np.array_equal(gk2[d], gk[s])
    pageable = torch.zeros((4, heads, B, D), dtype=tdt)
    with pytest.raises(ValueError):
        pa.pa_swap_blocks(pageable, pageable, k, v, _d32([0]), _d32([1]))
    ids = _d32([0])
    rc = pa.load_library().pa_swap_blocks(pageable.data_ptr(), pageable.data_ptr(), k.data_ptr(),
                                          v.data_ptr(), ids.data_ptr(), ids.data_ptr(), 1, NG, 4,
                                          heads, D, B, 1 if dtype == "bf16" else 0, None)
    assert rc == 1, "the library must refuse pageable host memory"
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(k), gk2)


@pytest.mark.parametrize("path", ["kernel", "dma"])
def test_layer_pipelined_swap_in_decode(path):
    """Four layers of a GQA decode batch whose K/V live in a pinned host tier:
    layer i+1 is swapped into one of two GPU layer pools on a copy stream
    while layer i's attention runs on the compute stream (events order the
    reuse of each pool).  kernel: pa_swap_blocks reads the host tier across
    the link; dma: pa_swap_in_staged moves the layer's blocks as one
    contiguous pinned run with the copy engines, then scatters them.  Every
    layer's output against the oracle run on that layer's host pool."""
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import attention_ref
    from workloads import build_workload
    L, hq, hkv = 4, 32, 8
    layers = [build_workload(f"swap layer {i}", 60 + i, dtype="bf16", num_q_heads=hq,
                             num_kv_heads=hkv, cached_lens=[700, 1500, 33, 2047, 900, 260],
                             new_lens=[1] * 6, pool_factor=1.25, placement="contiguous")
              for i in range(L)]
    wl0 = layers[0]
    NB = wl0.num_blocks
    assert all(w.num_blocks == NB and np.array_equal(w.block_tables, wl0.block_tables)
               for w in layers)
    # Host tier: every layer's pool, written once (the new tokens included),
    # its blocks in order; the GPU pools get them scattered.
    from oracle import kv_write_ref
    host_np = [kv_write_ref(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping)
               for w in layers]
    tdt = torch_dtype("bf16")

    def pinned(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).pin_memory()

    host = [(pinned(kp), pinned(vp)) for kp, vp in host_np]
    # The GPU pools hold a layer's blocks under other ids: host block b -> pi[b].
    pi = np.random.default_rng(61).permutation(NB)
    used = np.unique(wl0.block_tables[wl0.block_tables >= 0])
    src_ids, dst_ids = _d32(used), _d32(pi[used])
    gpu_tab = np.where(wl0.block_tables >= 0, pi[np.maximum(wl0.block_tables, 0)], -1)
    bufs = [(torch.full((NB, hkv, B, D), float("nan"), dtype=tdt, device="cuda"),
             torch.full((NB, hkv, B, D), float("nan"), dtype=tdt, device="cuda"))
            for _ in range(2)]
    q = [_d16(w.q, "bf16") for w in layers]
    tab, lens, qsl = _d32(gpu_tab), _d32(wl0.context_lens), _d32(wl0.query_start_loc)
    outs = [torch.empty_like(x) for x in q]
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    landed = [torch.cuda.Event() for _ in range(L)]
    done = [torch.cuda.Event() for _ in range(L)]

    # dma: each layer's blocks as one contiguous pinned run in the order of
    # `used`, staged on the device, then scattered to pi[used].
    runs = [(pinned(kp[used]), pinned(vp[used])) for kp, vp in host_np]
    staging = [(torch.empty((used.size, hkv, B, D), dtype=tdt, device="cuda"),
                torch.empty((used.size, hkv, B, D), dtype=tdt, device="cuda")) for _ in range(2)]

    def swap_in(i):
        with torch.cuda.stream(copy):
            if i >= 2:
                copy.wait_event(done[i - 2])     # that pool's previous layer is finished
            k, v = bufs[i % 2]
            if path == "kernel":
                pa.pa_swap_blocks(k, v, host[i][0], host[i][1], src_ids, dst_ids, stream=copy)
            else:
                sk, sv = staging[i % 2]
                pa.pa_swap_in_staged(k, v, runs[i][0], runs[i][1], sk, sv, dst_ids, stream=copy)
            landed[i].record(copy)

    swap_in(0)
    for i in range(L):
        if i + 1 < L:
            swap_in(i + 1)
        compute.wait_event(landed[i])
        k, v = bufs[i % 2]
        pa.pa_attention(q[i], k, v, tab, lens, qsl, hkv, D ** -0.5, max_query_len=1,
                        max_context_len=wl0.max_context_len, out=outs[i], stream=compute)
        done[i].record(compute)
    torch.cuda.synchronize()
    for i, w in enumerate(layers):
        kp, vp = host_np[i]
        ref, _ = attention_ref(w.q, kp, vp, w.block_tables, w.context_lens, w.query_start_loc,
                               hkv, w.scale, "bf16")
        assert_close(host_bits(outs[i]), ref, "bf16", what=f"pipelined swap-in ({path}), layer {i}")


def test_staged_swap_out_and_in_round_trip():
    """Pool blocks swapped out through a staging run into a contiguous pinned
    host run, then swapped back in under other ids: bit for bit."""
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import swap_blocks_ref
    rng = np.random.default_rng(77)
    NB, H = 150, 8
    gk = rng.integers(0, 65536, size=(NB, H, B, D), dtype=np.uint16)
    gv = rng.integers(0, 65536, size=(NB, H, B, D), dtype=np.uint16)
    k, v = _d16(gk, "bf16"), _d16(gv, "bf16")
    tdt = torch_dtype("bf16")
    out_ids = rng.permutation(NB)[:60]
    hk = torch.empty((60, H, B, D), dtype=tdt).pin_memory()
    hv = torch.empty((60, H, B, D), dtype=tdt).pin_memory()
    sk = torch.empty((64, H, B, D), dtype=tdt, device="cuda")
    sv = torch.empty((64, H, B, D), dtype=tdt, device="cuda")
    pa.pa_swap_out_staged(hk, hv, k, v, sk, sv, _d32(out_ids))
    torch.cuda.synchronize()
    run_k, run_v = swap_blocks_ref(np.zeros((60, H, B, D), np.uint16),
                                   np.zeros((60, H, B, D), np.uint16), gk, gv, out_ids,
                                   np.arange(60))
    assert np.array_equal(hk.view(torch.int16).numpy().view(np.uint16), run_k)
    assert np.array_equal(hv.view(torch.int16).numpy().view(np.uint16), run_v)
    back = rng.permutation(NB)[:60]
    pa.pa_swap_in_staged(k, v, hk, hv, sk, sv, _d32(back))
    torch.cuda.synchronize()
    gk2, gv2 = swap_blocks_ref(gk, gv, run_k, run_v, np.arange(60), back)
    assert np.array_equal(host_bits(k), gk2) and np.array_equal(host_bits(v), gv2)

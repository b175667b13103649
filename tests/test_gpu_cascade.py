"""Shared-prefix decode (cascade) vs the CPU oracle, through the C ABI.

Decode sequences whose block tables begin with the same physical blocks
(prefix sharing through identical table entries, PagedAttention explainer,
"メモリ共有") have the common blocks attended once for the whole group by the
matrix-core kernel; each member's decode then covers its own tail and merges
the group's (max, sum, output) records.  These tests check the outputs
against the fp64 oracle, and read back from the workspace which groups the
kernel formed, against a host model of the grouping rule, so that a silent
fall-back to plain decode cannot pass for the cascade.
"""
import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, to_dev
from ws_layout import workspace_layout
from workloads import build_workload
from workloads.configs import c4

pytestmark = pytest.mark.gpu

MIN_BLOCKS = 4        # shared blocks needed before a group forms
MAX_MEMBERS = 32      # members per group (and at most 128 rows: 128 // G)
PREFIX_CHUNKS = 8     # workgroups per (group, KV head) at most
CHUNK_TILES = 16      # 64-key tiles of the shared range per workgroup, at least


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()


def expected_groups(wl):
    """(shared blocks, chunks) per sequence under the grouping rule."""
    S = wl.num_seqs
    G = wl.num_q_heads // wl.num_kv_heads
    n = np.diff(wl.query_start_loc)
    C = wl.context_lens
    tab = wl.block_tables
    shareable = (C.astype(np.int64) - 1) // 16

    def linked(x):
        return (1 <= x < S and n[x] == 1 and n[x - 1] == 1 and shareable[x] >= MIN_BLOCKS
                and shareable[x - 1] >= MIN_BLOCKS
                and np.array_equal(tab[x, :MIN_BLOCKS], tab[x - 1, :MIN_BLOCKS]))

    max_members = min(MAX_MEMBERS, 128 // G)
    out = np.zeros((S, 2), dtype=np.int64)
    if S and int(n.max()) * G > 8:
        return out  # a call that may prefill runs no shared-prefix pass
    s = 0
    groups = []
    while s < S:
        # s starts a group when no link reaches it or its run hits the member cap
        members = 1
        while members < max_members and linked(s + members):
            members += 1
        groups.append((s, members))
        s += members
    for lead, members in groups:
        if members == 1:
            continue
        rows = tab[lead:lead + members]
        cap = int(shareable[lead:lead + members].min())
        same = np.all(rows[:, :cap] == rows[0, :cap], axis=0)
        shared = int(np.argmin(same)) if not same.all() else cap
        tiles = -(-shared * 16 // 64)
        chunks = min(PREFIX_CHUNKS, max(1, tiles // CHUNK_TILES))
        out[lead:lead + members] = (shared, chunks)
    return out


def _workspace_starts(wl, ws):
    """The [S][2] starts region of a workspace after a call; also checks that
    the call left the plan's item count and the decode's counters at zero."""
    S = wl.num_seqs
    lay = workspace_layout(S, wl.num_q_heads, wl.num_kv_heads, wl.max_context_len,
                           wl.max_query_len)
    assert lay["total"] == ws.numel() or ws.numel() == 1
    zero = ws[:lay["zero_bytes"]].cpu().numpy()
    assert not zero.any(), "the item count and counters are left at zero"
    if not lay["cascade"]:
        return np.zeros((S, 2), dtype=np.int32)
    raw = ws[lay["starts"]:lay["starts"] + S * 8].cpu().numpy().view(np.int32)
    return raw.reshape(S, 2)


def _run(wl, d, write=True):
    import torch
    import paged_kv_cache_14_amd as pa
    if write:
        pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    need = pa.pa_attention_workspace_size(wl.num_seqs, wl.total_q, wl.num_q_heads,
                                          wl.num_kv_heads, 128, wl.max_context_len,
                                          wl.max_query_len)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    out = pa.pa_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"],
                          d["context_lens"], d["query_start_loc"], wl.num_kv_heads, wl.scale,
                          max_query_len=wl.max_query_len, max_context_len=wl.max_context_len,
                          workspace=ws)
    torch.cuda.synchronize()
    return out, ws


def _check(wl, what, bare=False):
    d = to_dev(wl)
    out, ws = _run(wl, d)
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    exp = expected_groups(wl)
    got = _workspace_starts(wl, ws)
    assert np.array_equal(got, exp), f"{what}: groups differ\n{np.c_[got, exp]}"
    err = assert_close(host_bits(out), ref, wl.dtype, bare=bare, what=what)
    print(f"{what}: {int((exp[:, 0] > 0).sum())} of {wl.num_seqs} sequences grouped, "
          f"max|err| = {err:.3e}")
    return exp


def share_first_blocks(wl, x, k):
    """Point the first k table entries of sequence x at sequence x-1's blocks."""
    wl.block_tables[x, :k] = wl.block_tables[x - 1, :k]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_c4_shape_groups(dtype):
    # 3 prompts x 8 samples, 32 query / 8 KV heads, 512-token prefix; tails of
    # 0 keep the newest key in the last shared block
    wl = c4(21, prompts=3, samples=8, prefix=512, tail_hi=100, q_heads=32, kv_heads=8,
            dtype=dtype)
    exp = _check(wl, f"c4 shape {dtype}")
    assert (exp[:, 0] > 0).all()


@pytest.mark.parametrize("prefix,chunks", [(512, 1), (4096, 4)])
def test_whole_pair_dealing_with_one_and_four_prefix_chunks(prefix, chunks):
    # the shared-prefix GQA workload's scale (256 sequences, 8 KV heads, tails
    # up to 33 blocks), so that the decode deals whole pairs; a pair's first
    # two prefix records are loaded with its K/V, and with more than two
    # chunks the rest are folded from memory at its end
    wl = c4(29, prompts=32, samples=8, prefix=prefix, tail_hi=512, q_heads=32, kv_heads=8,
            dtype="bf16")
    exp = _check(wl, f"whole pairs, {prefix}-token prefix", bare=True)
    assert (exp[:, 1] == chunks).all()


def test_runs_longer_than_a_wave_and_the_member_cap():
    # 70 samples of one prompt, MHA: groups of 32, 32 and 6; the run behind the
    # last ones is longer than 64 sequences
    wl = c4(22, prompts=1, samples=70, prefix=128, tail_hi=40, q_heads=2, kv_heads=2,
            dtype="f16")
    exp = _check(wl, "70 samples")
    assert (exp[:, 0] == 8).sum() + (exp[:, 0] == 7).sum() == 70


def test_group_of_eight_heads_partial_tile():
    # G = 8: at most 16 members; 13 shared blocks = 3.25 tiles of 64 keys
    wl = c4(23, prompts=2, samples=20, prefix=208, tail_hi=60, q_heads=16, kv_heads=2,
            dtype="bf16")
    _check(wl, "G8 partial tile")


def test_split_tails_merge_with_prefix():
    # long tails: the decode splits them over many partitions, the first one
    # cut at the shared boundary, and the last to finish merges the prefix too
    wl = c4(24, prompts=2, samples=8, prefix=1024, tail_hi=3000, q_heads=4, kv_heads=2,
            dtype="bf16")
    _check(wl, "split tails")


def _partial_sharing(seq7_rows):
    cached = [300, 300, 300, 300, 80, 68, 500, 40, 500, 500, 700, 700, 64, 64, 900, 900]
    new = [1, 1, 1, 1, 1, 1, 1, seq7_rows, 1, 2, 1, 1, 1, 1, 1, 1]
    wl = build_workload("partial", 25, dtype="bf16", num_q_heads=8, num_kv_heads=2,
                        cached_lens=cached, new_lens=new, pool_factor=1.3)
    share_first_blocks(wl, 1, 18)   # 18 shared blocks
    share_first_blocks(wl, 2, 7)    # the group keeps 7
    share_first_blocks(wl, 3, 3)    # 3 < 4: 3 starts its own group
    share_first_blocks(wl, 4, 5)    # 3 and 4 share 5 blocks
    share_first_blocks(wl, 5, 4)    # 5 (C = 69: 4 shareable) joins with 4 blocks
    share_first_blocks(wl, 6, 4)    # 6 (C = 501) joins, the group keeps 4
    share_first_blocks(wl, 8, 2)    # 7 has several query rows: no link into 8
    share_first_blocks(wl, 9, 10)   # 9 has two query rows: no link
    share_first_blocks(wl, 11, 40)  # 10 and 11 share 40 blocks
    share_first_blocks(wl, 13, 4)   # C = 65: exactly 4 shareable blocks each
    wl.block_tables[15, :56] = wl.block_tables[14, :56]
    wl.block_tables[15, 30] = wl.block_tables[14, 31]  # differs from block 30 on
    return wl


def test_partial_sharing_decode_batch():
    """Sharing of various lengths between neighbours, broken by speculative
    sequences and by contexts too short to share."""
    wl = _partial_sharing(2)
    exp = _check(wl, "partial sharing")
    assert exp[:3, 0].tolist() == [7, 7, 7]
    assert exp[3:7, 0].tolist() == [4, 4, 4, 4]
    assert exp[7:10, 0].tolist() == [0, 0, 0]
    assert exp[10:12, 0].tolist() == [40, 40]
    assert exp[12:14, 0].tolist() == [4, 4]
    assert exp[14:16, 0].tolist() == [30, 30]


def test_call_that_may_prefill_runs_no_shared_prefix_pass():
    """The same tables with sequence 7 a 20-token prefill run: the call may
    prefill, so no sequence is grouped (the decode sequences read their shared
    blocks themselves), and every output still matches the oracle."""
    wl = _partial_sharing(20)
    lay = workspace_layout(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads, wl.max_context_len,
                           wl.max_query_len)
    assert lay["prefill"] and not lay["cascade"]
    exp = _check(wl, "sharing in a call that may prefill")
    assert not exp.any()


def test_no_sharing_leaves_the_plain_decode():
    """Without shared tables the cascade pass writes zero starts, so the decode
    covers every block as the plain path does: the batch and the same
    sequences one at a time (no cascade) all match the oracle, and a repeat
    of the batch call gives the same bits (the split depends on the batch,
    never on timing: a merge folds the slices in order whichever ends last)."""
    wl = build_workload("noshare", 26, dtype="f16", num_q_heads=8, num_kv_heads=2,
                        cached_lens=[900, 200, 1500, 77], new_lens=[1, 1, 1, 1],
                        pool_factor=1.2)
    d = to_dev(wl)
    out, ws = _run(wl, d)
    assert not _workspace_starts(wl, ws).any()
    ref, kp, vp = oracle_full(wl)
    got = host_bits(out)
    assert_close(got, ref, wl.dtype, what="no sharing, batch")
    out2, _ = _run(wl, d, write=False)
    assert np.array_equal(host_bits(out2), got), "repeat call differs"
    import paged_kv_cache_14_amd as pa
    import torch
    for s in range(wl.num_seqs):
        q0, q1 = int(wl.query_start_loc[s]), int(wl.query_start_loc[s + 1])
        o = pa.pa_attention(d["q"][q0:q1].contiguous(), d["k_pool"], d["v_pool"],
                            d["block_tables"][s:s + 1].contiguous(),
                            d["context_lens"][s:s + 1].contiguous(),
                            torch.tensor([0, q1 - q0], dtype=torch.int32, device="cuda"),
                            wl.num_kv_heads, wl.scale, max_query_len=q1 - q0,
                            max_context_len=wl.max_context_len)
        torch.cuda.synchronize()
        assert_close(host_bits(o), ref[q0:q1], wl.dtype, what=f"sequence {s} alone")


def test_cascade_repeat_calls_reuse_workspace():
    """The starts region is rewritten by every call: a grouped workload followed
    by an ungrouped one on the same workspace, and back."""
    import torch
    import paged_kv_cache_14_amd as pa
    a = c4(27, prompts=2, samples=4, prefix=256, tail_hi=30, q_heads=8, kv_heads=2)
    b = c4(28, prompts=2, samples=4, prefix=256, tail_hi=30, q_heads=8, kv_heads=2)
    # b: break every link (the tables keep their data, only sharing stops)
    nb = b.num_blocks
    extra = []
    for s in range(b.num_seqs):
        for j in range(16):
            extra.append(b.block_tables[s, j])
            b.block_tables[s, j] = nb + len(extra) - 1
    b.k_pool = np.concatenate([b.k_pool, b.k_pool[extra]])
    b.v_pool = np.concatenate([b.v_pool, b.v_pool[extra]])
    refs = [oracle_full(w)[0] for w in (a, b)]
    devs = [to_dev(w) for w in (a, b)]
    for w, d in zip((a, b), devs):
        pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    mc = max(a.max_context_len, b.max_context_len)
    need = pa.pa_attention_workspace_size(a.num_seqs, a.total_q, 8, 2, 128, mc, 1)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for rep in range(4):
        i = rep % 2
        w, d = (a, b)[i], devs[i]
        out = pa.pa_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"],
                              d["context_lens"], d["query_start_loc"], 2, w.scale,
                              max_query_len=1, max_context_len=mc, workspace=ws)
        torch.cuda.synchronize()
        assert_close(host_bits(out), refs[i], "bf16", what=f"call {rep}")


def test_workspace_reused_after_a_prefill_only_call():
    """A workspace zero-filled once serves a prefill-only call (GQA group of
    16: no decode rows, only the prefill's work queues) and then a
    shared-prefix decode with as many (sequence, KV head) pairs.  The zero
    region sits in front of every call's other regions, so the decode finds
    its item count at zero where the prefill's queues would otherwise have
    left their final heads."""
    import torch
    import paged_kv_cache_14_amd as pa
    pf = build_workload("pf16", 41, dtype="bf16", num_q_heads=16, num_kv_heads=1,
                        cached_lens=[300, 500, 64, 900], new_lens=[40, 17, 100, 9],
                        pool_factor=1.3)
    dec = c4(42, prompts=1, samples=2, prefix=256, tail_hi=40, q_heads=8, kv_heads=2)
    assert pf.num_seqs * pf.num_kv_heads == dec.num_seqs * dec.num_kv_heads == 4
    lay_pf = workspace_layout(pf.num_seqs, 16, 1, pf.max_context_len, pf.max_query_len)
    assert lay_pf["prefill"] and lay_pf["rows"] == 0 and lay_pf["zero_bytes"] == 512
    needs = [pa.pa_attention_workspace_size(w.num_seqs, w.total_q, w.num_q_heads,
                                            w.num_kv_heads, 128, w.max_context_len,
                                            w.max_query_len) for w in (pf, dec)]
    ws = torch.zeros(max(needs), dtype=torch.uint8, device="cuda")
    outs = []
    for w in (pf, dec):
        d = to_dev(w)
        pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
        outs.append(pa.pa_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"],
                                    d["context_lens"], d["query_start_loc"], w.num_kv_heads,
                                    w.scale, max_query_len=w.max_query_len,
                                    max_context_len=w.max_context_len, workspace=ws))
        torch.cuda.synchronize()
    for w, out, what in zip((pf, dec), outs, ("prefill-only", "shared-prefix decode after it")):
        assert_close(host_bits(out), oracle_full(w)[0], w.dtype, what=what)
    lay = workspace_layout(dec.num_seqs, 8, 2, dec.max_context_len, 1)
    assert lay["cascade"]
    got = ws[lay["starts"]:lay["starts"] + dec.num_seqs * 8].cpu().numpy().view(np.int32)
    assert np.array_equal(got.reshape(-1, 2), expected_groups(dec)), "the decode grouped its samples"
    assert not ws[:lay["zero_bytes"]].cpu().numpy().any(), "zero region left at zero"

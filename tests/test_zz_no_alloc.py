"""pa_attention_noalloc (static per-GPU scratch, no allocation) against
pa_attention on a caller workspace, through the C ABI, on an MI355X.

Two calls in a row, the second with a smaller batch, each checked bit for bit
against pa_attention's output (same kernels, same plan) and against the fp64
oracle at 2e-3 + half an ulp; a call larger than the scratch array holds is
rejected before anything is enqueued.
"""
import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, to_dev
from workloads import build_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()


# (name, dtype, Hq, Hkv, cached, new): decode with split pairs and shared-prefix
# planning, then a smaller mixed decode + prefill batch
CALLS = [
    ("big decode bf16", "bf16", 8, 2, [3000, 1500, 700, 20, 2600, 64], [1, 1, 1, 1, 1, 1]),
    ("small mixed bf16", "bf16", 8, 2, [40, 300], [24, 1]),
]


def _both(wl):
    import torch
    import paged_kv_cache_14_amd as pa
    d = to_dev(wl)
    pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    ref_out = pa.pa_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"],
                              d["context_lens"], d["query_start_loc"], wl.num_kv_heads, wl.scale,
                              max_query_len=wl.max_query_len,
                              max_context_len=wl.max_context_len)
    out = torch.full_like(d["q"], float("nan"))
    pa.pa_attention_noalloc(d["q"], d["k_pool"], d["v_pool"], d["block_tables"],
                            d["context_lens"], d["query_start_loc"], wl.num_kv_heads, wl.scale,
                            out=out, max_query_len=wl.max_query_len,
                            max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    return host_bits(ref_out), host_bits(out)


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    for name, dtype, hq, hkv, cached, new in CALLS:
        print(f"[no-alloc] {name}", flush=True)
        wl = build_workload(name, 77, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                            cached_lens=cached, new_lens=new, pool_factor=1.3)
        want, got = _both(wl)
        assert np.array_equal(got, want), f"{name}: differs from pa_attention"
        ref, _, _ = oracle_full(wl)
        assert_close(got, ref, dtype, what=f"no-alloc {name}")


# the wide prefill's two forms (its queues and ranking live in the workspace
# too): 1600 rows per KV head (4-wave form), then 400 (8-wave form)
WIDE_CALLS = [
    ("wide 4-wave f16", "f16", 16, 2, [2100, 30], [200, 1]),
    ("wide 8-wave bf16", "bf16", 16, 4, [1200, 64, 5], [100, 60, 1]),
]


def test_noalloc_matches_workspace_entry_point_on_wide_prefill_calls():
    for name, dtype, hq, hkv, cached, new in WIDE_CALLS:
        print(f"[no-alloc] {name}", flush=True)
        wl = build_workload(name, 78, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                            cached_lens=cached, new_lens=new, pool_factor=1.3)
        want, got = _both(wl)
        assert np.array_equal(got, want), f"{name}: differs from pa_attention"
        ref, _, _ = oracle_full(wl)
        assert_close(got, ref, dtype, what=f"no-alloc {name}")


def test_noalloc_rejects_calls_beyond_the_scratch_array():
    import torch
    import paged_kv_cache_14_amd as pa
    # 70000 one-token sequences x 1 KV head: more counters than the zero region holds
    S = 70000
    q = torch.zeros((S, 1, 128), dtype=torch.float16, device="cuda")
    pool = torch.zeros((4, 1, 16, 128), dtype=torch.float16, device="cuda")
    tables = torch.zeros((S, 1), dtype=torch.int32, device="cuda")
    lens = torch.ones(S, dtype=torch.int32, device="cuda")
    qsl = torch.arange(S + 1, dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(pa.PaError, match="ESCRATCH"):
        pa.pa_attention_noalloc(q, pool, pool, tables, lens, qsl, 1, 0.088, out=out,
                                max_query_len=1, max_context_len=1)
    torch.cuda.synchronize()
    assert not out.any()

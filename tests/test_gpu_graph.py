"""A step captured into a HIP graph replays correctly, on an MI355X.

The library enqueues only kernels: no memset, no allocation, no host read
when the caller passes the output, the workspace and the two host bounds.
Its per-call state (the shared-prefix plan's item count, the decode's merge
counters, the prefill's queues) returns to zero inside the kernels, so a
captured pa_kv_write + pa_attention can be replayed.  Each case captures one
step, replays it three times with eager work and synchronisations in
between, and checks every replay against the fp64 oracle.
"""
import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, to_dev
from workloads import build_workload
from workloads.configs import c4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()  # fails loudly if the HIP library is not built


def _replays(wl, what):
    import torch
    import paged_kv_cache_14_amd as pa
    d = to_dev(wl)
    ref, kp, vp = oracle_full(wl)
    out = torch.empty_like(d["q"])
    need = pa.pa_attention_workspace_size(wl.num_seqs, wl.total_q, wl.num_q_heads,
                                          wl.num_kv_heads, 128, wl.max_context_len,
                                          wl.max_query_len)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")

    def step():
        pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
        pa.pa_attention(d["q"], d["k_pool"], d["v_pool"], d["block_tables"], d["context_lens"],
                        d["query_start_loc"], wl.num_kv_heads, wl.scale,
                        max_query_len=wl.max_query_len, max_context_len=wl.max_context_len,
                        out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager step before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert_close(host_bits(out), ref, wl.dtype, what=f"{what}, eager")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(d["k_pool"]), kp), f"{what}: pool after replay {i}"
        err = assert_close(host_bits(out), ref, wl.dtype, what=f"{what}, replay {i}")
    print(f"{what}: 3 replays, max|err| = {err:.3e}")


def test_shared_prefix_step_replays():
    # plan + shared-prefix pass + decode with merged prefix records
    wl = c4(41, prompts=3, samples=6, prefix=320, tail_hi=200, q_heads=8, kv_heads=2,
            dtype="bf16")
    _replays(wl, "shared prefix")


def test_mixed_decode_prefill_step_replays():
    # decode slices cut across waves (merge counters), short pairs, prefill
    # queues and order, speculative rows
    cached = [3000, 12, 900, 0, 4500, 40]
    new = [1, 1, 30, 100, 1, 3]
    wl = build_workload("graph mixed", 42, dtype="f16", num_q_heads=8, num_kv_heads=2,
                        cached_lens=cached, new_lens=new, pool_factor=1.3)
    _replays(wl, "mixed")

"""The decode's equal-slice work split, against the fp64 oracle, on an MI355X.

The decode cuts the batch's (sequence, KV head, block) units into equal
slices, one per wave; sequences are read in windows of 64.  These cases reach
the parts of that split the configuration shapes do not: many windows (and
more windows than a wave keeps sums of), sequences without decode work mixed
in (prefill rows, no rows), long (sequence, head) pairs cut into many slices
beside short ones that are never cut, and a single wave.
"""
import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, run_step, to_dev
from workloads import build_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()  # fails loudly if the HIP library is not built


def _check(wl, what):
    import torch
    d = to_dev(wl)
    out = run_step(wl, d)
    torch.cuda.synchronize()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    err = assert_close(host_bits(out), ref, wl.dtype, what=what)
    print(f"{what}: {wl.num_seqs} sequences, max|err| = {err:.3e}")


@pytest.mark.parametrize("dtype,hq,hkv", [("f16", 2, 2), ("bf16", 8, 2)])
def test_five_windows_with_idle_sequences(dtype, hq, hkv):
    # 300 sequences (5 windows of 64); every 7th prefills (n*G > 8), every
    # 11th has no query rows
    rng = np.random.default_rng(301)
    S = 300
    cached = rng.integers(1, 400, size=S)
    G = hq // hkv
    new = np.ones(S, dtype=np.int64)
    new[::7] = 9 // G + 1
    new[5::11] = 0
    wl = build_workload("five windows", 302, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                        cached_lens=cached, new_lens=new, pool_factor=1.2)
    _check(wl, f"five windows {dtype} {hq}/{hkv}")


def test_more_windows_than_kept_sums():
    # 4200 sequences = 66 windows: past the 64 window sums a wave keeps, it
    # recounts the windows it walks over
    rng = np.random.default_rng(303)
    S = 4200
    cached = rng.integers(1, 40, size=S)
    wl = build_workload("66 windows", 304, dtype="bf16", num_q_heads=1, num_kv_heads=1,
                        cached_lens=cached, new_lens=np.ones(S, dtype=np.int64),
                        pool_factor=1.2)
    _check(wl, "66 windows")


@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 4, 4), ("f16", 16, 4)])
def test_long_pairs_cut_beside_short_ones(dtype, hq, hkv):
    # Two long sequences cut into many slices each (more records per merge
    # than one fetch round), between sequences shorter than a slice
    cached = [15, 20000, 3, 40, 9000, 1, 100, 64]
    wl = build_workload("long and short", 305, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                        cached_lens=cached, new_lens=[1] * len(cached), pool_factor=1.2)
    _check(wl, f"long and short {dtype} {hq}/{hkv}")


def test_one_wave_takes_the_batch():
    # 4 units: a grid of one wave, no counters or records in the workspace
    import paged_kv_cache_14_amd as pa
    wl = build_workload("one wave", 306, dtype="f16", num_q_heads=1, num_kv_heads=1,
                        cached_lens=[63], new_lens=[1], pool_factor=1.5)
    assert pa.pa_attention_workspace_size(1, 1, 1, 1, 128, 64, 1) == 0
    _check(wl, "one wave")


@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 32, 8), ("f16", 16, 16)])
def test_short_pairs_dealt_whole(dtype, hq, hkv):
    # 400 decode sequences of at most 10 blocks: the grid's equal slice (the
    # batch's units over 1024 or 2048 waves) is longer than the longest
    # pair, so whole pairs are dealt longest first in snake order
    rng = np.random.default_rng(305)
    S = 400
    cached = rng.integers(0, 160, size=S)
    wl = build_workload("snake", 306, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                        cached_lens=cached, new_lens=np.ones(S, dtype=np.int64),
                        pool_factor=1.2)
    T = -(-wl.context_lens.astype(np.int64) // 16)
    waves = 1024 if hq // hkv >= 4 else 2048
    assert T.max() <= T.sum() * hkv // waves  # the condition for whole pairs
    _check(wl, f"snake {dtype} {hq}/{hkv}")

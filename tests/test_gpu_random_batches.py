"""Seeded random batches against the fp64 oracle, every output compared.

Each batch mixes what one pa_attention call can hold: decode tokens, a few
speculative rows, runs of new prefill tokens (causal among themselves, full
attention to the cached history), empty sequences, and groups of one-token
samples that share their leading blocks through identical table entries
(PagedAttention explainer, "Copy-on-Writeによるメモリ共有" and "Prefix
Caching").  Head counts, grouping, lengths and the element type are drawn
per batch, so the calls cross every routing boundary of the library: the
decode on the vector ALUs (1-2 rows per KV head) and on the matrix cores
(4-8), the shared-prefix plan and pass, the narrow prefill (at most 128 rows
per KV head) and both forms of the wide prefill.  The tolerance is 2e-3 plus
half an output ulp (short contexts give |out| near 1 and more).
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


def random_batch(seed):
    """One seeded batch: (workload, a short description)."""
    rng = np.random.default_rng(10_000 + seed)
    dtype = "bf16" if rng.random() < 0.5 else "f16"
    hkv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    # kinds of sequences in this batch: decode always, the others by chance
    kinds = ["decode"]
    if rng.random() < 0.4:
        kinds.append("spec")
    if rng.random() < 0.5:
        kinds.append("prefill")
    if rng.random() < 0.15:
        kinds.append("empty")
    cached, new = [], []
    groups = []
    n_seqs = int(rng.integers(1, 11))
    for _ in range(n_seqs):
        kind = kinds[int(rng.integers(len(kinds)))]
        c = int(rng.integers(0, 2500)) if rng.random() < 0.9 else int(rng.integers(0, 40))
        if kind == "decode":
            n = 1
        elif kind == "spec":
            n = int(rng.integers(2, 9))
        elif kind == "prefill":
            n = int(rng.integers(9, 300))
        else:
            n = 0
        cached.append(c)
        new.append(n)
    prefix_blocks = 0
    if rng.random() < 0.35:
        # a group of one-token samples sharing their first blocks
        members = int(rng.integers(2, 10))
        prefix_blocks = int(rng.integers(4, 60))
        first = len(cached)
        for _ in range(members):
            cached.append(prefix_blocks * 16 + int(rng.integers(0, 200)))
            new.append(1)
        groups.append(list(range(first, first + members)))
    wl = build_workload(f"random {seed}", 20_000 + seed, dtype=dtype, num_q_heads=hkv * g,
                        num_kv_heads=hkv, cached_lens=cached, new_lens=new, pool_factor=1.3,
                        shared_prefix_groups=groups or None,
                        shared_prefix_blocks=prefix_blocks)
    what = (f"batch {seed}: {dtype}, {hkv * g}/{hkv} heads, {len(cached)} sequences, "
            f"query lengths {new}, {'a group sharing ' + str(prefix_blocks) + ' blocks' if groups else 'no sharing'}")
    return wl, what


@pytest.mark.parametrize("seed", range(40))
def test_random_batch(seed):
    import torch
    wl, what = random_batch(seed)
    if wl.total_q == 0:
        pytest.skip("no query rows drawn")
    d = to_dev(wl)
    out = run_step(wl, d)
    torch.cuda.synchronize()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    assert np.array_equal(host_bits(d["v_pool"]), vp)
    assert_close(host_bits(out), ref, wl.dtype, what=what)


def random_long_batch(seed):
    """A seeded batch for the wide kernel's steady steps: prefill runs of
    129-400 tokens over cached contexts of 1024-6000 keys, so that items see
    at least 1024 keys and round the weights of their steady range."""
    rng = np.random.default_rng(30_000 + seed)
    dtype = "bf16" if rng.random() < 0.75 else "f16"
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    n_seqs = int(rng.integers(2, 6))
    cached = [int(rng.integers(1024, 6000)) for _ in range(n_seqs)]
    new = [int(rng.integers(129, 401)) if rng.random() < 0.7 else 1 for _ in range(n_seqs)]
    wl = build_workload(f"random long {seed}", 40_000 + seed, dtype=dtype, num_q_heads=hkv * g,
                        num_kv_heads=hkv, cached_lens=cached, new_lens=new, pool_factor=1.2)
    return wl, (f"long batch {seed}: {dtype}, {hkv * g}/{hkv} heads, cached {cached}, "
                f"query lengths {new}")


@pytest.mark.parametrize("seed", range(16))
def test_random_long_batch(seed):
    import torch
    wl, what = random_long_batch(seed)
    d = to_dev(wl)
    out = run_step(wl, d)
    torch.cuda.synchronize()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    assert_close(host_bits(out), ref, wl.dtype, what=what)

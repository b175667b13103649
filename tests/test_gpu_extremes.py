"""Sizes at the ends of what the library takes, against the fp64 oracle, every
output compared.

- One decode sequence of 131,072 (GQA 32/8) or 65,536 (MHA) tokens: its
  (sequence, KV head) pairs are cut into a few hundred slices, and the last
  slice of each folds all their records (PagedAttention explainer,
  "PagedAttentionアルゴリズム": the blockwise form of the attention equation).
- 128 query heads over 16 KV heads (G = 8, the most rows the decode takes per
  KV head), in a decode batch and in a call that also prefills.
- 64 KV heads, MHA, decode and prefill rows mixed.
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


def _check(wl, what, bare=False):
    import torch
    d = to_dev(wl)
    out = run_step(wl, d)
    torch.cuda.synchronize()
    ref, kp, vp = oracle_full(wl)
    assert np.array_equal(host_bits(d["k_pool"]), kp)
    assert np.array_equal(host_bits(d["v_pool"]), vp)
    err = assert_close(host_bits(out), ref, wl.dtype, bare=bare, what=what)
    print(f"{what}: {wl.num_seqs} sequences, {int(wl.context_lens.max())} longest context, "
          f"max|err| = {err:.3e}")


@pytest.mark.parametrize("dtype,hq,hkv,ctx", [("bf16", 32, 8, 131072), ("f16", 8, 8, 65536)],
                         ids=["gqa_131072", "mha_65536"])
def test_one_long_context_decode(dtype, hq, hkv, ctx):
    # the newest token is written by kv_write first, as in a decode step
    wl = build_workload(f"long {ctx}", 401 + hkv, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                        cached_lens=[ctx - 1], new_lens=[1], pool_factor=1.1)
    _check(wl, f"one {ctx}-token decode, {hq}/{hkv} heads, {dtype}", bare=True)


def test_long_context_decode_beside_short_ones():
    # a 65,536-token sequence among short ones: its slices and the short
    # sequences' whole pairs in one grid
    cached = [65535, 17, 300, 1, 4000, 63]
    wl = build_workload("long beside short", 407, dtype="bf16", num_q_heads=16, num_kv_heads=4,
                        cached_lens=cached, new_lens=[1] * len(cached), pool_factor=1.1)
    # (2e-3 plus half an output ulp: a 2-key sequence gives |out| near 2)
    _check(wl, "65,536 tokens beside short sequences")


def test_128_query_heads_over_16_kv_heads_decode():
    rng = np.random.default_rng(408)
    S = 48
    cached = rng.integers(0, 3000, size=S)
    wl = build_workload("128/16 decode", 408, dtype="bf16", num_q_heads=128, num_kv_heads=16,
                        cached_lens=cached, new_lens=np.ones(S, dtype=np.int64), pool_factor=1.2)
    _check(wl, "128/16 heads decode")


def test_128_query_heads_over_16_kv_heads_with_prefill():
    cached = [700, 0, 2500, 129, 40]
    new = [1, 37, 1, 200, 5]
    wl = build_workload("128/16 mixed", 409, dtype="f16", num_q_heads=128, num_kv_heads=16,
                        cached_lens=cached, new_lens=new, pool_factor=1.3)
    _check(wl, "128/16 heads, decode and prefill")


def test_64_kv_heads_mha_mixed():
    cached = [1000, 64, 3000, 0, 515]
    new = [1, 1, 90, 33, 1]
    wl = build_workload("64 heads", 410, dtype="bf16", num_q_heads=64, num_kv_heads=64,
                        cached_lens=cached, new_lens=new, pool_factor=1.3)
    _check(wl, "64 MHA heads, decode and prefill")

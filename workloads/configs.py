"""The five seeded workloads paged attention is measured and checked on.

Each builder draws its lengths from ``numpy.random.default_rng`` seeded with
the workload's seed, then hands them to :func:`build_workload`.  Integer
ranges are inclusive.  Every decode step first writes its newest token's K/V
(``pa_kv_write``) and then attends over all ``C`` keys, the new one included;
when that newest key sits in a block other sequences share, it is already
cached and nothing is written (slot ``-1``).

* ``c1`` single-sequence decode: 1 query, 512 keys, 8 heads, fp16, the 32
  blocks at a random permutation of a 64-block pool.
* ``c2`` batched decode on a Llama-2-13B-like MHA layer: 64 sequences,
  ``C ~ U[128, 4096]``, 40 heads, fp16, pool 1.2x the need, shuffled free list.
* ``c3`` multi-turn prefill: 32 sessions, cached ``~U[1024, 8192]``, new
  ``~U[16, 256]`` (causal among themselves, full view of the cache), 40 heads,
  bf16, pool 1.2x, new K/V written first.
* ``c4`` GQA decode with shared prefixes: 32 prompts x 8 samples, 32 query /
  8 KV heads, bf16; each prompt's 8 samples share its 128 prefix blocks
  (2048 tokens) through identical block-table entries; private tails
  ``~U[0, 512]``.
* ``c5`` long-context chunked prefill, GQA: 4 sequences with 32768 cached and
  2048 new causal tokens each, 64 query / 8 KV heads, bf16, fully random
  placement in a pool 1.1x the need.
"""
from __future__ import annotations

import numpy as np

from .generate import BLOCK_SIZE, PagedWorkload, build_workload

CONFIG_NAMES = ("c1", "c2", "c3", "c4", "c5")

DESCRIPTIONS = {
    "c1": "single-sequence decode, 512 keys, 8 heads, fp16",
    "c2": "batched decode, 64 seqs, C~U[128,4096], 40 heads MHA (Llama-2-13B-like layer), fp16",
    "c3": "multi-turn prefill, 32 sessions, cached~U[1024,8192], new~U[16,256], 40 heads, bf16",
    "c4": "GQA 32/8 decode, 32 prompts x 8 samples, 2048-token shared prefix + tail~U[0,512], bf16",
    "c5": "GQA 64/8 chunked prefill, 4 seqs x (32768 cached + 2048 new), bf16",
}


def c1(seed: int = 1, *, contexts: int = 512, heads: int = 8, pool_blocks: int = 64,
       dtype: str = "f16") -> PagedWorkload:
    return build_workload(
        "c1", seed, dtype=dtype, num_q_heads=heads, num_kv_heads=heads,
        cached_lens=[contexts - 1], new_lens=[1], num_blocks=pool_blocks)


def c2(seed: int = 2, *, num_seqs: int = 64, lo: int = 128, hi: int = 4096, heads: int = 40,
       dtype: str = "f16", placement: str = "shuffled") -> PagedWorkload:
    rng = np.random.default_rng(seed)
    C = rng.integers(lo, hi, size=num_seqs, endpoint=True)
    return build_workload(
        "c2", seed, dtype=dtype, num_q_heads=heads, num_kv_heads=heads,
        cached_lens=C - 1, new_lens=np.ones(num_seqs, dtype=np.int64), pool_factor=1.2,
        placement=placement)


def c3(seed: int = 3, *, num_seqs: int = 32, cached_lo: int = 1024, cached_hi: int = 8192,
       new_lo: int = 16, new_hi: int = 256, heads: int = 40, dtype: str = "bf16",
       placement: str = "shuffled") -> PagedWorkload:
    rng = np.random.default_rng(seed)
    cached = rng.integers(cached_lo, cached_hi, size=num_seqs, endpoint=True)
    new = rng.integers(new_lo, new_hi, size=num_seqs, endpoint=True)
    return build_workload(
        "c3", seed, dtype=dtype, num_q_heads=heads, num_kv_heads=heads,
        cached_lens=cached, new_lens=new, pool_factor=1.2, placement=placement)


def c4(seed: int = 4, *, prompts: int = 32, samples: int = 8, prefix: int = 2048,
       tail_hi: int = 512, q_heads: int = 32, kv_heads: int = 8,
       dtype: str = "bf16") -> PagedWorkload:
    assert prefix % BLOCK_SIZE == 0
    rng = np.random.default_rng(seed)
    tails = rng.integers(0, tail_hi, size=prompts * samples, endpoint=True)
    C = prefix + tails
    groups = [list(range(p * samples, (p + 1) * samples)) for p in range(prompts)]
    return build_workload(
        "c4", seed, dtype=dtype, num_q_heads=q_heads, num_kv_heads=kv_heads,
        cached_lens=C - 1, new_lens=np.ones_like(C), pool_factor=1.2,
        shared_prefix_groups=groups, shared_prefix_blocks=prefix // BLOCK_SIZE,
        new_in_pool=(tails == 0))


def c5(seed: int = 5, *, num_seqs: int = 4, cached: int = 32768, new: int = 2048,
       q_heads: int = 64, kv_heads: int = 8, dtype: str = "bf16",
       placement: str = "shuffled") -> PagedWorkload:
    return build_workload(
        "c5", seed, dtype=dtype, num_q_heads=q_heads, num_kv_heads=kv_heads,
        cached_lens=np.full(num_seqs, cached), new_lens=np.full(num_seqs, new),
        pool_factor=1.1, placement=placement)


BUILDERS = {"c1": c1, "c2": c2, "c3": c3, "c4": c4, "c5": c5}
DEFAULT_SEEDS = {"c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}


def make_config(name: str, seed: int | None = None, **overrides) -> PagedWorkload:
    """Full-size workload ``name`` (``"c1"`` .. ``"c5"``); ``overrides`` shrink it."""
    if name not in BUILDERS:
        raise KeyError(f"unknown workload {name!r}; expected one of {CONFIG_NAMES}")
    return BUILDERS[name](DEFAULT_SEEDS[name] if seed is None else seed, **overrides)

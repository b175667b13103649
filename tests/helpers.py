"""Test-side helpers: lay logical (contiguous) K/V out in a paged pool.

The layout code here is written independently of ``oracle/`` so that a
mistake in the oracle's gather cannot cancel against the same mistake here.
"""
from __future__ import annotations

import numpy as np

from workloads import normal_bits

B = 16


def to_f64(bits, dtype):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def from_f64(x, dtype):
    """Exactly representable float64 values -> 16-bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f16":
        out = x.astype(np.float16)
        assert np.array_equal(out.astype(np.float64), x), "value not exact in f16"
        return out.view(np.uint16)
    f = x.astype(np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0) and np.array_equal(f.astype(np.float64), x), \
        "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def paged_layout(logical_k, logical_v, num_blocks, rng, pad=-1, placement="shuffled"):
    """Place per-sequence logical K/V ``[C_s, Hkv, D]`` (bit patterns) in a pool.

    Returns (k_pool, v_pool, block_tables); unused slots and blocks hold NaN.
    """
    S = len(logical_k)
    Hkv, D = logical_k[0].shape[1], logical_k[0].shape[2]
    need = [-(-k.shape[0] // B) for k in logical_k]
    assert sum(need) <= num_blocks
    order = rng.permutation(num_blocks) if placement == "shuffled" else np.arange(num_blocks)
    nan = np.uint16(0x7E00)
    k_pool = np.full((num_blocks, Hkv, B, D), nan, dtype=np.uint16)
    v_pool = np.full((num_blocks, Hkv, B, D), nan, dtype=np.uint16)
    tables = np.full((S, max(need) if need else 1), pad, dtype=np.int32)
    nxt = 0
    for s in range(S):
        for j in range(need[s]):
            tables[s, j] = order[nxt]
            nxt += 1
        for pos in range(logical_k[s].shape[0]):
            blk = tables[s, pos // B]
            k_pool[blk, :, pos % B, :] = logical_k[s][pos]
            v_pool[blk, :, pos % B, :] = logical_v[s][pos]
    return k_pool, v_pool, tables


def random_case(seed, ctx, new, hq, hkv, dtype="f16", d=128, pool_extra=3):
    """Logical K/V, q bits and metadata for a tiny random case."""
    ss = np.random.SeedSequence(seed)
    a, b, c, e = ss.spawn(4)
    rng = np.random.default_rng(e)
    lk = [normal_bits(np.random.SeedSequence([seed, 1, s]), (C, hkv, d), dtype)
          for s, C in enumerate(ctx)]
    lv = [normal_bits(np.random.SeedSequence([seed, 2, s]), (C, hkv, d), dtype)
          for s, C in enumerate(ctx)]
    nb = sum(-(-C // B) for C in ctx) + pool_extra
    k_pool, v_pool, tables = paged_layout(lk, lv, nb, rng)
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = normal_bits(c, (int(qsl[-1]), hq, d), dtype)
    return dict(q=q, k_pool=k_pool, v_pool=v_pool, block_tables=tables,
                context_lens=np.asarray(ctx, dtype=np.int32), query_start_loc=qsl,
                num_kv_heads=hkv, lk=lk, lv=lv, dtype=dtype)


def brute_force(q_bits, lk, lv, ctx, qsl, hkv, scale, dtype):
    """softmax(scale QK^T + bottom-right causal mask) V over contiguous logical K/V.

    Uses torch's CPU scaled_dot_product_attention in float64 with an explicit
    boolean mask (a library routine, independent of the oracle).
    """
    import torch
    Tq, Hq, D = q_bits.shape
    G = Hq // hkv
    out = np.zeros((Tq, Hq, D))
    for s in range(len(ctx)):
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        n, C = hi - lo, int(ctx[s])
        if n == 0:
            continue
        K = torch.from_numpy(to_f64(lk[s], dtype))          # [C, Hkv, D]
        V = torch.from_numpy(to_f64(lv[s], dtype))
        Q = torch.from_numpy(to_f64(q_bits[lo:hi], dtype))  # [n, Hq, D]
        rows = torch.arange(n)[:, None]
        cols = torch.arange(C)[None, :]
        allowed = cols <= (C - n + rows)
        for h in range(Hq):
            o = torch.nn.functional.scaled_dot_product_attention(
                Q[:, h][None], K[:, h // G][None], V[:, h // G][None],
                attn_mask=allowed[None], scale=scale)
            out[lo:hi, h] = o[0].numpy()
    return out

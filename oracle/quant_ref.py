"""Plain CPU model of quantized KV pages -- TEST INFRASTRUCTURE ONLY.

Only ``tests/`` import this module; the product path (libpa's page encoder
and its decode over quantized pages) never calls it and shares no code with
it.

What it computes, and where the pages define it (KV-cache textbook ch.22,
the Kitty passage):

* K and V are stored at 2 bits per value.  Key channels differ in how much
  quantization hurts them: a few channels carry consistently large
  magnitudes.  The channels with the largest mean magnitude over the group's
  tokens get 4 bits instead of 2 (the text's range is the top 12.5% to 25%;
  taken here: 12.5%, 16 of 128 channels).
* A quantization group of 128 tokens is one page, so quantized pages stay
  compatible with paged attention; a page is quantized once, when its 128
  tokens are complete (the heavy work amortized over 128 decode steps).
* A promoted channel's 4-bit code is its low 2 bits, kept in the dense plane
  every channel has, plus its high 2 bits, kept in a small sparse plane of
  only the promoted channels (so every channel is read the same way).

Readings of what the passage leaves open (the library takes the same ones,
as a convention, not as code):

* Keys are quantized per channel along the page's 128 tokens; values per
  token along its 128 channels (the KIVI arrangement the chapter names).
* Asymmetric uniform quantization: for a group g of values x, mn = min x,
  mx = max x, scale = (mx - mn) / (2^bits - 1) and
  code = min(2^bits - 1, rint((x - mn) / scale)), every step in float32
  with round-to-nearest-even (code 0 when scale is 0); the value it stands
  for is mn + code * scale.  The decision of a code is integer work taken in
  the precision both sides use, float32, so codes and parameters are
  bit-exact.
* Promotion ranks channels by the float32 sum of |k| over the page's tokens,
  accumulated in token order; ties go to the lower channel index.
* The tokens of a sequence's last, unfinished page stay unquantized (16-bit)
  in the block pool.
"""
from __future__ import annotations

import numpy as np

PAGE_TOKENS = 128
BOOST_CHANNELS = 16   # 12.5% of 128 channels get 4-bit codes


def _f32_values(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of fp16 / bf16 bit patterns."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def quantize_groups(x: np.ndarray, levels, axis: int):
    """(codes uint8, scale float32, mn float32) of the groups of float32 values
    that run along `axis` of x (one group per index of the other axis);
    `levels` is 3 or 15 per group."""
    x = np.asarray(x, dtype=np.float32)
    mn = x.min(axis=axis).astype(np.float32)
    mx = x.max(axis=axis).astype(np.float32)
    lv = np.broadcast_to(np.asarray(levels, dtype=np.float32), mn.shape)
    scale = ((mx - mn) / lv).astype(np.float32)
    e_mn = np.expand_dims(mn, axis)
    e_sc = np.expand_dims(scale, axis)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((x - e_mn) / e_sc).astype(np.float32)
    q = np.where(e_sc == 0, np.float32(0), q)
    codes = np.minimum(q, np.expand_dims(lv, axis)).astype(np.uint8)
    return codes, scale, mn


def boosted_channels(k_vals: np.ndarray, count: int = BOOST_CHANNELS) -> np.ndarray:
    """The `count` channels with the largest float32 sum of |k| over the page's
    tokens (a running sum in token order), ties to the lower index; ascending."""
    sums = np.cumsum(np.abs(k_vals), axis=0, dtype=np.float32)[-1]
    # stable sort of -sum keeps the lower index first among equal sums
    order = np.argsort(-sums.astype(np.float64), kind="stable")
    return np.sort(order[:count])


def quantize_page(k_bits: np.ndarray, v_bits: np.ndarray, dtype: str) -> dict:
    """One page (128 tokens x 128 channels of one KV head) -> its logical
    quantized form: per-channel K codes (2 or 4 bits), per-token V codes."""
    k = _f32_values(k_bits, dtype)
    v = _f32_values(v_bits, dtype)
    T, D = k.shape
    assert T == PAGE_TOKENS and v.shape == (T, D)
    boost = boosted_channels(k)
    levels = np.full(D, 3, dtype=np.float32)
    levels[boost] = 15
    k_codes, k_scale, k_min = quantize_groups(k, levels, axis=0)   # per channel
    v_codes, v_scale, v_min = quantize_groups(v, 3, axis=1)        # per token
    return dict(boost=boost, k_codes=k_codes, k_scale=k_scale, k_min=k_min,
                v_codes=v_codes, v_scale=v_scale, v_min=v_min)


def dequantize_page(page: dict):
    """(K, V) [128, 128] float64: mn + code * scale, exactly."""
    k = page["k_min"].astype(np.float64)[None, :] + \
        page["k_codes"].astype(np.float64) * page["k_scale"].astype(np.float64)[None, :]
    v = page["v_min"].astype(np.float64)[:, None] + \
        page["v_codes"].astype(np.float64) * page["v_scale"].astype(np.float64)[:, None]
    return k, v


def attention_quant_ref(q: np.ndarray, pages, k_pool: np.ndarray, v_pool: np.ndarray,
                        block_tables: np.ndarray, context_lens: np.ndarray,
                        quant_lens: np.ndarray, query_start_loc: np.ndarray,
                        num_kv_heads: int, scale: float, dtype: str) -> np.ndarray:
    """fp64 attention of every query row over its sequence's keys, the first
    quant_lens[s] of them read from quantized pages and the rest from the
    16-bit pool through the block table.

    ``pages[s][g]`` is the list of logical pages (``quantize_page`` output) of
    sequence s, KV head g, covering its first quant_lens[s] tokens.  Row i of
    n new rows sees keys 0 .. C - n + i (bottom-right causal).
    """
    from .paged_ref import _softmax_attend, bits_to_f64
    Tq, Hq, D = q.shape
    G = Hq // num_kv_heads
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    for s in range(len(context_lens)):
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        n, C, Q = hi - lo, int(context_lens[s]), int(quant_lens[s])
        assert 0 <= n <= C and 0 <= Q <= C and Q % PAGE_TOKENS == 0
        if n == 0:
            continue
        for g in range(num_kv_heads):
            ks, vs = [], []
            for p in pages[s][g]:
                kk, vv = dequantize_page(p)
                ks.append(kk)
                vs.append(vv)
            assert len(ks) * PAGE_TOKENS == Q
            for j in range(Q // 16, -(-C // 16)):
                phys = int(block_tables[s, j])
                ks.append(bits_to_f64(k_pool[phys, g], dtype))
                vs.append(bits_to_f64(v_pool[phys, g], dtype))
            K = np.concatenate(ks)[:C] if ks else np.zeros((0, D))
            V = np.concatenate(vs)[:C] if vs else np.zeros((0, D))
            rows = np.arange(n)
            limit = C - n + rows
            for h in range(g * G, (g + 1) * G):
                Qh = bits_to_f64(q[lo:hi, h], dtype)
                o, _, _ = _softmax_attend(Qh, K, V, scale, limit)
                out[lo:hi, h] = o
    return out

"""Checks that tie the quantized-page model of the oracle to the textbook's
description (KV-cache textbook ch.22, Kitty) and to mathematics.

Each ``pin_*`` takes the model's module (``oracle.quant_ref`` or a copy with
a planted mistake) and raises ``AssertionError`` on disagreement.
"""
from __future__ import annotations

import math

import numpy as np

from helpers import B, brute_force, from_f64, paged_layout, to_f64

T = 128
D = 128


def _levels_page(rng, dtype):
    """K whose every channel takes values on 4 equally spaced levels, V whose
    every token does.  Steps are 5 * 2^-k, so the 2-bit step (span / 3 = the
    step) and the 4-bit one (span / 15 = step / 5) are exact in float32 and
    both reproduce the data exactly."""
    k = np.zeros((T, D))
    for c in range(D):
        base, step = rng.integers(-8, 8) / 4, 5 * 2.0 ** -rng.integers(3, 6)
        k[:, c] = base + step * rng.integers(0, 4, size=T)
        k[0, c], k[1, c] = base, base + 3 * step           # both ends present
    v = np.zeros((T, D))
    for t in range(T):
        base, step = rng.integers(-8, 8) / 4, 5 * 2.0 ** -rng.integers(3, 6)
        v[t] = base + step * rng.integers(0, 4, size=D)
        v[t, 0], v[t, 1] = base, base + 3 * step
    return from_f64(k, dtype), from_f64(v, dtype), k, v


def pin_exact_on_four_levels(o):
    """Data on 4 equally spaced levels per group round-trips exactly."""
    rng = np.random.default_rng(1)
    for dtype in ("f16", "bf16"):
        kb, vb, k, v = _levels_page(rng, dtype)
        kk, vv = o.dequantize_page(o.quantize_page(kb, vb, dtype))
        assert np.array_equal(kk, k) and np.array_equal(vv, v)


def pin_error_within_half_a_step(o):
    """Every value is within half its group's step (plus float32 rounding)."""
    rng = np.random.default_rng(2)
    kb = from_f64(rng.standard_normal((T, D)).astype(np.float16), "f16")
    vb = from_f64(rng.standard_normal((T, D)).astype(np.float16), "f16")
    p = o.quantize_page(kb, vb, "f16")
    kk, vv = o.dequantize_page(p)
    k, v = to_f64(kb, "f16"), to_f64(vb, "f16")
    tol_k = p["k_scale"].astype(np.float64)[None, :] * (0.5 + 1e-5) + 1e-6
    tol_v = p["v_scale"].astype(np.float64)[:, None] * (0.5 + 1e-5) + 1e-6
    assert np.all(np.abs(kk - k) <= tol_k) and np.all(np.abs(vv - v) <= tol_v)
    # the ends of each group are represented exactly
    assert np.array_equal(p["k_min"].astype(np.float64), k.min(axis=0))
    assert np.array_equal(p["v_min"].astype(np.float64), v.min(axis=1))
    assert np.allclose(kk.max(axis=0), k.max(axis=0), rtol=0, atol=1e-5)


def pin_promoted_channels_are_the_largest(o):
    """The 16 channels of largest mean |k| get 4-bit codes; ties go to the
    lower index; the rest keep 2 bits."""
    rng = np.random.default_rng(3)
    k = rng.standard_normal((T, D))
    big = np.sort(rng.permutation(D)[:16])
    k[:, big] *= 10.0
    kb = from_f64(k.astype(np.float16), "f16")
    vb = from_f64(rng.standard_normal((T, D)).astype(np.float16), "f16")
    p = o.quantize_page(kb, vb, "f16")
    assert list(p["boost"]) == list(big)
    kvals = to_f64(kb, "f16")
    for c in range(D):
        levels = 15 if c in big else 3
        assert p["k_codes"][:, c].max() <= levels
        want = (kvals[:, c].max() - kvals[:, c].min()) / levels
        assert abs(float(p["k_scale"][c]) - want) <= 1e-6 * max(1.0, want)
    same = np.tile(np.arange(D, dtype=np.float64) % 3 - 1, (T, 1))   # |k| sums 0 or T
    p2 = o.quantize_page(from_f64(same, "f16"), vb, "f16")
    ones = [c for c in range(D) if c % 3 != 1]
    assert list(p2["boost"]) == ones[:16]


def pin_promotion_cuts_the_error(o):
    """A promoted channel's worst error is a fifth of what 2 bits leave."""
    rng = np.random.default_rng(4)
    kb = from_f64(rng.standard_normal((T, D)).astype(np.float16), "f16")
    vb = from_f64(rng.standard_normal((T, D)).astype(np.float16), "f16")
    p = o.quantize_page(kb, vb, "f16")
    kk, _ = o.dequantize_page(p)
    k = to_f64(kb, "f16")
    for c in p["boost"]:
        span = k[:, c].max() - k[:, c].min()
        assert np.max(np.abs(kk[:, c] - k[:, c])) <= span / 30 * (1 + 1e-5) + 1e-6


def _paged_with_pages(o, seed, ctx, new, hq, hkv, dtype, exact):
    """A batch whose first floor(C/128)*128 keys per sequence are quantized
    pages and the rest 16-bit blocks; returns everything the attention needs
    plus the logical (dequantized + tail) K/V for brute force."""
    rng = np.random.default_rng(seed)
    S = len(ctx)
    lk, lv = [], []
    for C in ctx:
        if exact:
            ks, vs = [], []
            for _ in range(-(-C // T)):
                kb, vb, _, _ = _levels_page(rng, dtype)
                ks.append(kb[:, None, :].repeat(hkv, axis=1))
                vs.append(vb[:, None, :].repeat(hkv, axis=1))
            lk.append(np.concatenate(ks)[:C])
            lv.append(np.concatenate(vs)[:C])
        else:
            lk.append(from_f64(rng.standard_normal((C, hkv, D)).astype(np.float16), dtype)
                      if dtype == "f16" else
                      from_f64(np.round(rng.standard_normal((C, hkv, D)) * 8) / 8, dtype))
            lv.append(from_f64(rng.standard_normal((C, hkv, D)).astype(np.float16), dtype)
                      if dtype == "f16" else
                      from_f64(np.round(rng.standard_normal((C, hkv, D)) * 8) / 8, dtype))
    nb = sum(-(-C // B) for C in ctx) + 2
    kp, vp, tab = paged_layout(lk, lv, nb, rng)
    quant = np.array([C // T * T for C in ctx], np.int32)
    pages = [[[o.quantize_page(lk[s][p * T:(p + 1) * T, g], lv[s][p * T:(p + 1) * T, g], dtype)
               for p in range(quant[s] // T)] for g in range(hkv)] for s in range(S)]
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = from_f64(np.round(rng.standard_normal((int(qsl[-1]), hq, D)) * 8) / 8, dtype) \
        if dtype == "bf16" else from_f64(rng.standard_normal((int(qsl[-1]), hq, D)).astype(np.float16), dtype)
    return dict(q=q, pages=pages, kp=kp, vp=vp, tab=tab, ctx=np.array(ctx, np.int32),
                quant=quant, qsl=qsl, lk=lk, lv=lv)


def pin_quantized_attention_matches_the_plain_oracle_on_exact_pages(o):
    """Pages holding data their codes reproduce exactly: the attention over
    pages + 16-bit tail equals the plain paged oracle (to 1e-12)."""
    from oracle import attention_ref
    for dtype in ("f16", "bf16"):
        c = _paged_with_pages(o, 5, [300, 128, 40, 256], [1, 3, 1, 2], 8, 2, dtype, exact=True)
        got = o.attention_quant_ref(c["q"], c["pages"], c["kp"], c["vp"], c["tab"], c["ctx"],
                                    c["quant"], c["qsl"], 2, 1 / math.sqrt(D), dtype)
        want, _ = attention_ref(c["q"], c["kp"], c["vp"], c["tab"], c["ctx"], c["qsl"], 2,
                                1 / math.sqrt(D), dtype)
        assert np.max(np.abs(got - want)) <= 1e-12, np.max(np.abs(got - want))


def pin_quantized_attention_brute_force(o):
    """Random data: the attention over pages + tail equals torch SDPA over the
    contiguous dequantized keys and values followed by the 16-bit tail."""
    c = _paged_with_pages(o, 6, [260, 129, 384], [1, 2, 1], 4, 2, "f16", exact=False)
    S, hkv = 3, 2
    lk_hat, lv_hat = [], []
    for s in range(S):
        Q = int(c["quant"][s])
        ks, vs = [], []
        for g in range(hkv):
            kq = [o.dequantize_page(p)[0] for p in c["pages"][s][g]]
            vq = [o.dequantize_page(p)[1] for p in c["pages"][s][g]]
            ktail = to_f64(c["lk"][s][Q:, g], "f16")
            vtail = to_f64(c["lv"][s][Q:, g], "f16")
            ks.append(np.concatenate(kq + [ktail]))
            vs.append(np.concatenate(vq + [vtail]))
        lk_hat.append(np.stack(ks, axis=1))
        lv_hat.append(np.stack(vs, axis=1))
    want = _sdpa_f64(c["q"], lk_hat, lv_hat, c["ctx"], c["qsl"], hkv, 1 / math.sqrt(D))
    got = o.attention_quant_ref(c["q"], c["pages"], c["kp"], c["vp"], c["tab"], c["ctx"],
                                c["quant"], c["qsl"], hkv, 1 / math.sqrt(D), "f16")
    assert np.max(np.abs(got - want)) <= 1e-12, np.max(np.abs(got - want))


def _sdpa_f64(q_bits, lk, lv, ctx, qsl, hkv, scale):
    import torch
    Tq, Hq, _ = q_bits.shape
    G = Hq // hkv
    out = np.zeros((Tq, Hq, D))
    for s in range(len(ctx)):
        lo, hi = int(qsl[s]), int(qsl[s + 1])
        n, C = hi - lo, int(ctx[s])
        K, V = torch.from_numpy(lk[s]), torch.from_numpy(lv[s])
        Q = torch.from_numpy(to_f64(q_bits[lo:hi], "f16"))
        allowed = torch.arange(C)[None, :] <= (C - n + torch.arange(n)[:, None])
        for h in range(Hq):
            o = torch.nn.functional.scaled_dot_product_attention(
                Q[:, h][None], K[:, h // G][None], V[:, h // G][None], attn_mask=allowed[None],
                scale=scale)
            out[lo:hi, h] = o[0].numpy()
    return out


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

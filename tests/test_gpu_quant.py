"""Quantized KV pages on an MI355X: pa_quantize_pages bit for bit against the
oracle's quantizer, and decode attention over quantized pages followed by
16-bit blocks (pa_attention_quant) against the oracle's attention over the
dequantized pages, within 2e-3.

The bytes of a page are read back through `unpack_page`, which restates the
library's page layout (the decode's lane order) on the host.
"""
import zlib

import numpy as np
import pytest

from gpu_util import assert_close, host_bits, oracle_full, to_dev, torch_dtype
from workloads import build_workload

pytestmark = pytest.mark.gpu
T = 128
D = 128
PAGE_BYTES = 10816


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_14_amd as pa
    pa.load_library()
    assert pa.PA_QPAGE_BYTES == PAGE_BYTES


def _lane_maps():
    """Index maps of the page's code planes (the library's layout, restated):
    for every (word, bit pair) of the K low, K high and V planes, the
    (token, channel) its low and high codes stand for."""
    klo, khi, vlo = [], [], []
    for st in range(4):
        for l in range(64):
            q, j = l >> 4, l & 15
            for w in range(4):
                word = (st * 64 + l) * 4 + w
                for i in range(8):
                    p = i & 3
                    H, m = w >> 1, 2 * (w & 1) + (i >> 2)
                    key = 32 * st + 8 * (j >> 2) + 4 * H + (j & 3)
                    ch = 32 * m + 8 * q + 2 * p
                    klo.append((word, i, key, ch, key, ch + 1))
                    t = 2 * w + (i >> 2)
                    vkey = 32 * st + 8 * q + 2 * p
                    vlo.append((word, i, vkey, 16 * t + j, vkey + 1, 16 * t + j))
            if l < 32:
                for i in range(8):
                    H, p = i >> 2, i & 3
                    key = 32 * st + 8 * (j >> 2) + 4 * H + (j & 3)
                    khi.append((st * 32 + l, i, key, 8 * q + 2 * p, key, 8 * q + 2 * p + 1))
    return [np.array(x, dtype=np.int64) for x in (klo, khi, vlo)]


_MAPS = None


def unpack_page(buf):
    """Logical form of one page's bytes (uint8 [10816]), per the layout: code
    planes of 32-bit words whose bit pair i holds one code at bits 2i and the
    next at bits 16 + 2i, in the matrix-core decode's operand order; key
    parameters per channel and value parameters per token in plain order."""
    global _MAPS
    if _MAPS is None:
        _MAPS = _lane_maps()
    klo, khi, vlo = _MAPS
    buf = np.ascontiguousarray(buf, dtype=np.uint8)

    def fields(words, m):
        w = words[m[:, 0]]
        sh = (2 * m[:, 1]).astype(np.uint32)
        return ((w >> sh) & 3).astype(np.uint8), ((w >> (sh + 16)) & 3).astype(np.uint8)

    boost = buf[5632:5648].astype(np.int64)
    k_codes = np.zeros((T, D), np.uint8)
    lo, hi = fields(buf[0:4096].view(np.uint32), klo)
    k_codes[klo[:, 2], klo[:, 3]] = lo
    k_codes[klo[:, 4], klo[:, 5]] = hi
    lo, hi = fields(buf[4096:4608].view(np.uint32), khi)
    k_codes[khi[:, 2], boost[khi[:, 3]]] += 4 * lo
    k_codes[khi[:, 4], boost[khi[:, 5]]] += 4 * hi
    v_codes = np.zeros((T, D), np.uint8)
    lo, hi = fields(buf[5696:9792].view(np.uint32), vlo)
    v_codes[vlo[:, 2], vlo[:, 3]] = lo
    v_codes[vlo[:, 4], vlo[:, 5]] = hi
    return dict(boost=boost, k_codes=k_codes, k_scale=buf[4608:5120].view(np.float32).copy(),
                k_min=buf[5120:5632].view(np.float32).copy(), v_codes=v_codes,
                v_scale=buf[9792:10304].view(np.float32).copy(),
                v_min=buf[10304:10816].view(np.float32).copy())


def _same_page(got, want, what):
    assert np.array_equal(got["boost"], want["boost"]), f"{what}: promoted channels"
    for key in ("k_codes", "v_codes"):
        assert np.array_equal(got[key], want[key]), f"{what}: {key}"
    for key in ("k_scale", "k_min", "v_scale", "v_min"):
        assert np.array_equal(got[key].view(np.uint32), want[key].view(np.uint32)), \
            f"{what}: {key}"


def _d32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quantize_pages_bit_exact(dtype):
    """Pages of N(0,1) data, a page whose 16 channels are 10x larger, one with
    constant channels and tokens (step 0), one whose |k| sums tie: codes,
    promoted channels and parameters bit for bit."""
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle.quant_ref import quantize_page
    from workloads.generate import _round_bits
    rng = np.random.default_rng(11 if dtype == "f16" else 12)
    Hkv, NB = 3, 64
    vals = rng.standard_normal((NB, Hkv, 16, D))
    vals[8:16, :, :, rng.permutation(D)[:16]] *= 10                    # page 1: heavy channels
    vals[16:24, :, :, :5] = 0.75                                       # page 2: constant channels
    vals[16:24, :, 3, :] = -1.5                                        # and constant tokens
    vals[24:32, :, :, :] = np.sign(vals[24:32]) * 0.5                  # page 3: |k| sums tie
    bits = _round_bits(vals.astype(np.float32), dtype)
    vbits = _round_bits(rng.standard_normal((NB, Hkv, 16, D)).astype(np.float32), dtype)
    tdt = torch_dtype(dtype)
    k = torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()
    v = torch.from_numpy(vbits.view(np.int16)).view(tdt).cuda()
    n = 6
    src = np.stack([rng.permutation(NB)[:8] for _ in range(2)] +
                   [np.arange(8 * p, 8 * p + 8) for p in range(4)]).astype(np.int32)
    page_ids = np.array([5, 0, 3, 1, 4, 2], np.int32)
    qpool = torch.zeros((n, Hkv, PAGE_BYTES), dtype=torch.uint8, device="cuda")
    pa.pa_quantize_pages(qpool, k, v, _d32(page_ids), _d32(src))
    torch.cuda.synchronize()
    got_pool = qpool.cpu().numpy()
    for i in range(n):
        for g in range(Hkv):
            kb = bits[src[i], g].reshape(T, D)
            vb = vbits[src[i], g].reshape(T, D)
            _same_page(unpack_page(got_pool[page_ids[i], g]), quantize_page(kb, vb, dtype),
                       f"page {i} head {g}")


def quant_setup(wl):
    """Each sequence's complete pages of cached keys (quant_lens = the largest
    multiple of 128 at most C - n), their blocks, and page ids in order."""
    qsl = wl.query_start_loc
    quant = np.array([(int(wl.context_lens[s]) - int(qsl[s + 1] - qsl[s])) // T * T
                      for s in range(wl.num_seqs)], np.int32)
    npg = quant // T
    max_pages = max(1, int(npg.max()))
    page_tables = np.full((wl.num_seqs, max_pages), -1, np.int32)
    src = []
    nxt = 0
    for s in range(wl.num_seqs):
        for p in range(npg[s]):
            page_tables[s, p] = nxt
            src.append(wl.block_tables[s, 8 * p:8 * p + 8])
            nxt += 1
    src = np.array(src, np.int32).reshape(-1, 8)
    return quant, page_tables, src, nxt


def oracle_pages(wl, kp, vp, quant, page_tables):
    from oracle.quant_ref import quantize_page
    pages = []
    for s in range(wl.num_seqs):
        per_head = []
        for g in range(wl.num_kv_heads):
            lst = []
            for p in range(int(quant[s]) // T):
                blocks = wl.block_tables[s, 8 * p:8 * p + 8]
                lst.append(quantize_page(kp[blocks, g].reshape(T, D), vp[blocks, g].reshape(T, D),
                                         wl.dtype))
            per_head.append(lst)
        pages.append(per_head)
    return pages


def run_quant(wl, check_pages=8):
    """kv_write, quantize the complete pages, decode over them; returns the
    output bits, the oracle's pools and pages, and the setup."""
    import torch
    import paged_kv_cache_14_amd as pa
    from oracle import kv_write_ref
    d = to_dev(wl)
    pa.pa_kv_write(d["k_new"], d["v_new"], d["k_pool"], d["v_pool"], d["slot_mapping"])
    quant, page_tables, src, npages = quant_setup(wl)
    qpool = torch.zeros((max(npages, 1), wl.num_kv_heads, PAGE_BYTES), dtype=torch.uint8,
                        device="cuda")
    if npages:
        pa.pa_quantize_pages(qpool, d["k_pool"], d["v_pool"],
                             _d32(np.arange(npages, dtype=np.int32)), _d32(src))
    out = pa.pa_attention_quant(d["q"], qpool, _d32(page_tables), _d32(quant), d["k_pool"],
                                d["v_pool"], d["block_tables"], d["context_lens"],
                                d["query_start_loc"], wl.num_kv_heads, wl.scale,
                                max_query_len=wl.max_query_len,
                                max_context_len=wl.max_context_len)
    torch.cuda.synchronize()
    kp, vp = kv_write_ref(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping)
    pages = oracle_pages(wl, kp, vp, quant, page_tables)
    got_pool = qpool.cpu().numpy()
    rng = np.random.default_rng(0)
    for _ in range(min(check_pages, npages)):     # a sample of pages, bit for bit
        s = int(rng.choice(np.flatnonzero(quant > 0)))
        p = int(rng.integers(quant[s] // T))
        g = int(rng.integers(wl.num_kv_heads))
        _same_page(unpack_page(got_pool[page_tables[s, p], g]), pages[s][g][p],
                   f"seq {s} page {p} head {g}")
    return host_bits(out), kp, vp, pages, quant


# (name, dtype, Hq, Hkv, cached_lens, new_lens): one decode instance each
CASES = [
    ("mha_f16", "f16", 4, 4, [0, 130, 1000, 5000, 256, 127], [1] * 6),
    ("gqa2_bf16", "bf16", 8, 4, [300, 2047, 128, 700], [1] * 4),
    ("gqa4_bf16", "bf16", 8, 2, [3000, 129, 511, 4100], [1] * 4),
    ("gqa8_f16", "f16", 16, 2, [900, 260, 2600], [1] * 3),
    ("speculative_gqa2_bf16", "bf16", 8, 4, [640, 1500, 255], [2, 3, 1]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_over_quantized_pages(case):
    from oracle import attention_ref
    from oracle.quant_ref import attention_quant_ref
    name, dtype, hq, hkv, cached, new = case
    wl = build_workload(name, zlib.crc32(name.encode()) % 10000, dtype=dtype, num_q_heads=hq,
                        num_kv_heads=hkv, cached_lens=cached, new_lens=new, pool_factor=1.3)
    got, kp, vp, pages, quant = run_quant(wl)
    ref = attention_quant_ref(wl.q, pages, kp, vp, wl.block_tables, wl.context_lens, quant,
                              wl.query_start_loc, hkv, wl.scale, dtype)
    assert_close(got, ref, dtype, what=f"quantized pages, {name}")
    exact, _ = attention_ref(wl.q, kp, vp, wl.block_tables, wl.context_lens,
                             wl.query_start_loc, hkv, wl.scale, dtype)
    print(f"[quant] {name}: 2-bit pages move the output by up to "
          f"{float(np.max(np.abs(ref - exact))):.3e} from the 16-bit oracle", flush=True)


def test_attention_over_quantized_pages_full_size_batched_decode():
    """The batched decode (64 sequences, contexts U[128, 4096], 40 heads,
    fp16) with every complete page of cached keys quantized: every output
    against the oracle at the bare 2e-3."""
    from oracle.quant_ref import attention_quant_ref
    from workloads import make_config
    wl = make_config("c2")
    print(f"[quant] full-size batched decode, {wl.num_seqs} sequences", flush=True)
    got, kp, vp, pages, quant = run_quant(wl, check_pages=32)
    ref = attention_quant_ref(wl.q, pages, kp, vp, wl.block_tables, wl.context_lens, quant,
                              wl.query_start_loc, wl.num_kv_heads, wl.scale, wl.dtype)
    assert_close(got, ref, wl.dtype, bare=True, what="quantized pages, full-size batched decode")

"""Closed forms against the numbers the pages print (tests/golden/closed_forms.json)."""
import json
import os

import pytest

import oracle.paged_ref as ref

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json"),
                        encoding="utf-8"))


def test_llama2_13b_bytes_per_token():
    g = GOLDEN["llama2_13b_kv_bytes_per_token"]
    b = ref.kv_bytes_per_token(g["layers"], g["hidden"], g["bytes_per_elem"])
    assert b == g["printed_bytes"]
    assert round(b / 2**20, 2) == g["printed_mb_approx"]


def test_llama2_13b_layer_of_the_batched_decode_workload():
    # one layer of 40 heads x 128 dims in fp16: 2 x 40 x 128 x 2 B per token;
    # 40 such layers give the page's per-token figure
    per_layer = ref.kv_bytes_per_token(1, 40 * 128, 2)
    assert per_layer == 20480
    assert 40 * per_layer == GOLDEN["llama2_13b_kv_bytes_per_token"]["printed_bytes"]


def test_gqa_group_4_quarter():
    g = GOLDEN["gqa_group4_fraction"]
    full = ref.kv_bytes_per_token(40, 5120, 2)
    grouped = ref.kv_bytes_per_token(40, 5120 // g["group_size"], 2)
    assert grouped / full == g["printed_fraction"]
    assert grouped == 204800


def test_40gb_holds_about_50000_tokens():
    g = GOLDEN["a100_40gb_token_capacity"]
    per = ref.kv_bytes_per_token(40, 5120, 2)
    for total in (g["kv_gb"] * 10**9, g["kv_gb"] * 2**30):
        tokens = total // per
        assert abs(tokens - g["printed_tokens_approx"]) <= 0.1 * g["printed_tokens_approx"]
    assert g["kv_gb"] * 10**9 // per == 48828
    assert g["kv_gb"] * 2**30 // per == 52428


def test_textbook_192_gib():
    g = GOLDEN["textbook_192gib"]
    elems = ref.kv_cache_elements(g["batch"], g["layers"], g["seq_len"], g["head_dim"], g["heads"])
    assert elems == 103_079_215_104
    assert elems * g["bytes_per_elem"] == g["printed_gib"] * 2**30


def test_opt13b_request_size():
    g = GOLDEN["opt13b_request"]
    for kb in (1000, 1024):
        for gb in (10**9, 2**30):
            size = g["printed_kb_per_token"] * kb * g["tokens"] / gb
            assert abs(size - g["printed_gb_per_request"]) <= 0.05 * g["printed_gb_per_request"]


@pytest.mark.parametrize("n,blocks,frag", [(0, 0, 0), (1, 1, 15), (15, 1, 1), (16, 1, 0),
                                           (17, 2, 15), (512, 32, 0), (34816, 2176, 0),
                                           (4095, 256, 1)])
def test_blocks_and_fragmentation(n, blocks, frag):
    assert GOLDEN["block_size_default"]["printed_block_size"] == ref.BLOCK_SIZE == 16
    assert ref.num_blocks(n) == blocks
    assert ref.internal_fragmentation(n) == frag
    assert 0 <= ref.internal_fragmentation(n) <= 15

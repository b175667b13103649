"""The quantized page's code planes, as the GPU test's unpacker restates them
(tests/test_gpu_quant.py, _lane_maps), cover every code exactly once.

A map that named one (token, channel) twice and another never would make the
encoder's bit-exact check compare the wrong codes without failing, so the
restatement is checked here on its own: each plane's (word, bit pair) slots
are used once and stay inside the plane, and their codes tile the page's
128 tokens x 128 channels (keys, low bits), 128 x 16 promoted slots (keys,
high bits) and 128 tokens x 128 dims (values).
"""
import numpy as np

from test_gpu_quant import _lane_maps


def _check(m, words, rows, cols):
    slots = m[:, 0] * 8 + m[:, 1]
    assert m[:, 0].min() >= 0 and m[:, 0].max() < words
    assert len(np.unique(slots)) == len(slots) == words * 8
    cover = np.zeros((rows, cols), np.int64)
    np.add.at(cover, (m[:, 2], m[:, 3]), 1)
    np.add.at(cover, (m[:, 4], m[:, 5]), 1)
    assert cover.min() == 1 and cover.max() == 1


def test_key_low_plane_covers_every_code_once():
    klo, _, _ = _lane_maps()
    _check(klo, 4096 // 4, 128, 128)


def test_key_high_plane_covers_every_promoted_slot_once():
    _, khi, _ = _lane_maps()
    _check(khi, 512 // 4, 128, 16)


def test_value_plane_covers_every_code_once():
    _, _, vlo = _lane_maps()
    _check(vlo, 4096 // 4, 128, 128)


def test_pairs_of_a_word_half_are_adjacent_channels_or_tokens():
    # the decode's code operand takes bit pair p of a word as the f16 pair
    # (element 2p, 2p+1): the two codes of a pair are adjacent channels (keys)
    # or adjacent tokens (values) of one row or dim
    klo, khi, vlo = _lane_maps()
    assert np.all(klo[:, 4] == klo[:, 2]) and np.all(klo[:, 5] == klo[:, 3] + 1)
    assert np.all(khi[:, 4] == khi[:, 2]) and np.all(khi[:, 5] == khi[:, 3] + 1)
    assert np.all(vlo[:, 5] == vlo[:, 3]) and np.all(vlo[:, 4] == vlo[:, 2] + 1)

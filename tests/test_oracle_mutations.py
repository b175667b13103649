"""Plant plausible mistakes in a copy of the oracle; some pin must catch each.

The mistakes are planted in the oracle's source text on the CPU (never in the
HIP path): a wrong causal alignment, a dropped scale or normalisation, a
wrong block lookup or slice, a swapped K/V, a wrong GQA head map, a dropped
rescale in the partition merge, a wrong bf16 decode, a wrong slot offset.
"""
import importlib.util
import os

import pytest

import oracle.paged_ref as ref
from oracle_pins import ALL_PINS

MUTATIONS = {
    "causal_top_left": ("return C - n + np.asarray(rows, dtype=np.int64)",
                        "return np.asarray(rows, dtype=np.int64)"),
    "causal_off_by_one": ("return C - n + np.asarray(rows, dtype=np.int64)",
                          "return C - n + np.asarray(rows, dtype=np.int64) - 1"),
    "dropped_scale": ("X = scale * (Q @ K.T)", "X = (Q @ K.T)"),
    "dropped_normalisation": ("W /= l\n", "W /= 1.0\n"),
    "logical_as_physical": ("phys = int(table_row[j])", "phys = j"),
    "wrong_partial_slice": ("K = np.concatenate(k_rows, axis=0)[:C]",
                            "K = np.concatenate(k_rows, axis=0)[-C:]"),
    "v_from_k_pool": ("v_rows.append(v_pool[phys, kv_head])",
                      "v_rows.append(k_pool[phys, kv_head])"),
    "interleaved_gqa": ("for h in range(g * G, (g + 1) * G):",
                        "for h in range(g, G * num_kv_heads, num_kv_heads):"),
    "merge_without_rescale": ("l_tot = sum(l * np.exp(m - M) for m, l, _ in live)",
                              "l_tot = sum(l for m, l, _ in live)"),
    "bf16_decode_shift": ("(bits.astype(np.uint32) << 16)", "(bits.astype(np.uint32) << 15)"),
    "kv_write_swapped": ("k_out[block, :, offset, :] = k_new[t]",
                         "k_out[block, :, offset, :] = v_new[t]"),
    "kv_write_offset": ("block, offset = divmod(slot, block_size)",
                        "block, offset = divmod(slot, block_size); offset = (offset + 1) % block_size"),
    "blockwise_drops_last_key": ("count = min(block_size, last_key + 1 - first)",
                                 "count = min(block_size, last_key - first)"),
    "sample_sequence_left": ('s = int(np.searchsorted(qsl, t, side="right") - 1)',
                             's = int(np.searchsorted(qsl, t, side="left") - 1)'),
    "sample_row_off_by_one": ("row = np.array([t - lo])", "row = np.array([t - lo + 1])"),
    "lse_wrong": ("return acc / l_tot, M + np.log(l_tot)", "return acc / l_tot, np.log(l_tot)"),
}


def _mutant(tmp_path, name, old, new):
    src = open(ref.__file__, encoding="utf-8").read()
    assert old in src, f"mutation {name} no longer applies"
    path = os.path.join(tmp_path, f"mutant_{name}.py")
    with open(path, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    mod = _mutant(str(tmp_path), name, *MUTATIONS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"

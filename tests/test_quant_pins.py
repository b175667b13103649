"""The oracle's quantized-page model against the textbook and mathematics,
and plausible mistakes planted in a copy of it, each caught by some pin."""
import importlib.util
import os

import pytest

import oracle.quant_ref as ref
from quant_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(ref)


MUTATIONS = {
    "boost_levels_three": ("    levels[boost] = 15\n", "    levels[boost] = 3\n"),
    "boost_smallest": ("order = np.argsort(-sums.astype(np.float64), kind=\"stable\")",
                       "order = np.argsort(sums.astype(np.float64), kind=\"stable\")"),
    "boost_ties_high_index": ("order = np.argsort(-sums.astype(np.float64), kind=\"stable\")",
                              "order = (len(sums) - 1 - np.argsort(-sums[::-1].astype(np.float64), kind=\"stable\"))"),
    "floor_not_round": ("q = np.rint(", "q = np.floor("),
    "v_per_channel": ("quantize_groups(v, 3, axis=1)", "quantize_groups(v, 3, axis=0)"),
    "dequant_drops_min": ("k = page[\"k_min\"].astype(np.float64)[None, :] + \\\n",
                          "k = 0 * page[\"k_min\"].astype(np.float64)[None, :] + \\\n"),
    "tail_one_block_late": ("for j in range(Q // 16, -(-C // 16)):",
                            "for j in range(Q // 16 + 1, -(-C // 16) + 1):"),
    "scale_off_by_one_level": ("scale = ((mx - mn) / lv).astype(np.float32)",
                               "scale = ((mx - mn) / (lv + 1)).astype(np.float32)"),
}


def _mutant(tmp_path, name, old, new):
    src = open(ref.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation {name} no longer applies"
    path = os.path.join(tmp_path, f"q_mutant_{name}.py")
    with open(path, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new).replace("from .paged_ref import", "from oracle.paged_ref import"))
    spec = importlib.util.spec_from_file_location(f"q_mutant_{name}", path)
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
        except (AssertionError, IndexError, ValueError, KeyError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"

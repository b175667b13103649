"""The oracle's block-management model against the pages and invariants, and
plausible mistakes planted in a copy of it, each caught by some pin."""
import importlib.util
import os

import pytest

import oracle.block_manager_ref as ref
from block_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(ref)


MUTATIONS = {
    "cow_only_at_three": ("and self.refcount[tab[-1]] >= 2:\n",
                          "and self.refcount[tab[-1]] >= 3:\n"),
    "cow_without_decrement": ("            self.refcount[old] -= 1\n", ""),
    "free_while_shared": ("            if self.refcount[b] == 0:\n",
                          "            if self.refcount[b] <= 1:\n"),
    "fork_without_reference": ("        for b in tab:\n            self.refcount[b] += 1\n"
                               "        self.tables.append(tab)\n        self.lengths.append(self.lengths[parent])",
                               "        self.tables.append(tab)\n        self.lengths.append(self.lengths[parent])"),
    "slot_offset": ("slots.append(tab[pos // BLOCK] * BLOCK + pos % BLOCK)",
                    "slots.append(tab[pos // BLOCK] * BLOCK + (pos + 1) % BLOCK)"),
    "free_list_as_stack": ("b = self.free.popleft()", "b = self.free.pop()"),
    "prefix_drops_partial_block": ("tab = self.table(src)[: -(-num_tokens // BLOCK)]",
                                   "tab = self.table(src)[: num_tokens // BLOCK]"),
    "copy_backwards": ("        k_out[d] = k_pool[s]\n", "        k_out[s] = k_pool[d]\n"),
    "swap_reads_destination": ("        k_out[d] = src_k[s]\n", "        k_out[d] = dst_k[s]\n"),
    "new_block_one_early": ("            if pos % BLOCK == 0:\n", "            if pos % BLOCK == 1:\n"),
}


def _mutant(tmp_path, name, old, new):
    src = open(ref.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation {name} no longer applies"
    path = os.path.join(tmp_path, f"bm_mutant_{name}.py")
    with open(path, "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"bm_mutant_{name}", path)
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
        except (AssertionError, IndexError, ValueError, KeyError, MemoryError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {name}"

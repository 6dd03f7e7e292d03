"""Pins for the swap space of the reference pool (oracle/pool.py, R7), and
planted mistakes that the pins must catch."""

import os
import types

import pytest

import swap_checks as sc
from oracle import RefPool, apply_append, ref_decode
from oracle.pool import apply_swap


def test_closed_forms():
    sc.check_swap_closed_forms(RefPool)


@pytest.mark.parametrize("seed", range(4))
def test_random_walk_against_unpaged_model(seed):
    sc.check_swap_against_unpaged_model(RefPool, apply_append, apply_swap, seed=seed)


def test_swap_round_trip_preserves_attention():
    sc.check_swap_preserves_attention(RefPool, apply_append, apply_swap, ref_decode)


ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

SWAP_MUTANTS = [
    ("shared blocks swapped out", "            if self._ref[b] == 1:\n                h = self._host_free.popleft()",
     "            if self._ref[b] >= 1:\n                h = self._host_free.popleft()"),
    ("swapped-out block not freed", "                self._ref[b] = 0\n                self._free.append(b)",
     "                self._ref[b] = 0"),
    ("swap-in keeps the host slot", "                copies.append((x, y))\n                self._host_free.append(x)",
     "                copies.append((x, y))"),
    ("free of a swapped sequence leaks slots", "                if kind == \"host\":\n                    self._host_free.append(x)",
     "                if kind == \"host\":\n                    pass"),
    ("swap-in takes from the back", "                y = self._free.popleft()\n                self._ref[y] = 1\n                copies.append((x, y))",
     "                y = self._free.pop()\n                self._ref[y] = 1\n                copies.append((x, y))"),
    ("copies run backwards", "        out[d] = src_pages[s]", "        out[s] = src_pages[d]"),
    ("host capacity not checked", "        if len(alone) > len(self._host_free):", "        if False:"),
]


@pytest.mark.parametrize("label,old,new", SWAP_MUTANTS, ids=[m[0] for m in SWAP_MUTANTS])
def test_swap_mutant_is_caught(label, old, new):
    src = open(os.path.join(ORACLE_DIR, "pool.py")).read()
    assert src.count(old) == 1, label
    mod = types.ModuleType("oracle_mutant_pool_swap")
    exec(compile(src.replace(old, new, 1), "pool.py", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        sc.run_swap_pins(mod.RefPool, mod.apply_append, mod.apply_swap, ref_decode)

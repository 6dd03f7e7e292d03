"""Pins for the prefix-cache oracle (oracle/radix.py): an independent flat model
of the cached block paths with brute-force matching and eviction choice, pool
reference accounting, and the pages' scenarios with closed-form outcomes."""

import pytest

import radix_checks as rc
from oracle import RefPool
from oracle.radix import RadixCache, RadixError


def test_system_prompt_shared_by_1000_users():
    hits = rc.scenario_system_prompt(RadixCache, RefPool)
    assert hits == 999 * 2000


def test_multi_turn_appends_to_previous_leaf():
    rc.scenario_multi_turn(RadixCache, RefPool)


def test_branch_and_backtrack():
    rc.scenario_branch_and_backtrack(RadixCache, RefPool)


def test_leaf_only_lru_eviction():
    rc.scenario_leaf_only_eviction(RadixCache, RefPool)


def test_evicting_blocks_still_in_use():
    rc.scenario_evict_blocks_in_use(RadixCache, RefPool)


def test_batched_admission():
    rc.scenario_batched_admission(RadixCache, RefPool)


def test_rsbcm_order():
    rc.scenario_rsbcm_order(RadixCache, RefPool)


@pytest.mark.parametrize("bs,num_blocks", [(1, 24), (2, 40), (4, 48)])
def test_random_traces_against_flat_model(bs, num_blocks):
    rc.run_traces(RadixCache, RefPool, seeds=(0, 1, 2), steps=250, bs=bs, num_blocks=num_blocks)


def test_partial_blocks_are_not_cached():
    pool = RefPool(8, 4)
    cache = RadixCache(pool)
    pool.alloc(0, 7)
    node, adopted = cache.insert(list(range(7)), pool.table(0))
    assert adopted == 1 and cache.node_tokens(node) == [0, 1, 2, 3]
    assert cache.match_prefix(list(range(7)))[0] == 4
    assert cache.match_prefix([0, 1, 2])[0] == 0


def test_errors():
    pool = RefPool(8, 2)
    cache = RadixCache(pool)
    with pytest.raises(RadixError):
        cache.insert([1, 2], [0])          # block 0 is free
    pool.alloc(0, 2)
    node, _ = cache.insert([1, 2], pool.table(0))
    with pytest.raises(RadixError):
        cache.unlock(node)                 # not locked
    with pytest.raises(KeyError):
        cache.lock(99)
    with pytest.raises(RadixError):
        cache.insert([1, 2], pool.table(0), score=float("nan"))
    with pytest.raises(RadixError):
        RadixCache(pool, "mru")


# -- planted mistakes (on the CPU): every one must fail the pins ---------------

import os
import types

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _load(module_file, old, new, imports):
    src = open(os.path.join(ORACLE_DIR, module_file)).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    src = src.replace(old, new, 1)
    for a, b in imports:
        src = src.replace(a, b)
    mod = types.ModuleType("oracle_mutant_" + module_file.replace(".", "_"))
    exec(compile(src, module_file, "exec"), mod.__dict__)
    return mod


RADIX_MUTANTS = [
    ("eviction ignores locks", "and not n.children and n.lock_ref == 0]", "and not n.children]"),
    ("eviction takes inner nodes", "and not n.children and n.lock_ref == 0]", "and n.lock_ref == 0]"),
    ("most recently used first", "victim = min(leaves, key=self.priority)", "victim = max(leaves, key=self.priority)"),
    ("match keeps the old time", "child.last_access_time = self.clock\n            blocks.extend(child.value)",
     "blocks.extend(child.value)"),
    ("lock only on the node", "for n in self._path(self._node(node_id)):\n            n.lock_ref += 1",
     "for n in self._path(self._node(node_id))[:1]:\n            n.lock_ref += 1"),
    ("split drops the lock", "upper.lock_ref = node.lock_ref", "upper.lock_ref = 0"),
    ("insert takes no reference", "self.pool.retain(b)", "pass"),
    ("eviction keeps the references", "if self.pool.release(b):", "if False:"),
    ("importance over depth + 2", "(node.depth + 1)", "(node.depth + 2)"),
    ("split hands over the wrong blocks", "node.key[:m], node.value[:m]", "node.key[:m], node.value[-m:]"),
    ("insert overwrites path scores", "child.score = max(child.score, float(score))", "child.score = float(score)"),
    ("match does not split", "                child = self._split(child, m)\n            child.last_access_time = self.clock\n            blocks.extend(child.value)",
     "                pass\n            child.last_access_time = self.clock\n            blocks.extend(child.value[:m])"),
    ("eviction stops one block early", "while released < num_blocks:", "while released < num_blocks - 1:"),
    ("score not raised on ancestors", "for n in self._path(node.parent):\n            n.score = max(n.score, float(score))",
     "for n in self._path(node.parent):\n            pass"),
    ("admission evicts nothing", "                self.evict(need - self.pool.free_count())",
     "                pass"),
    ("admission keeps the lock of a request that does not fit", "                self.unlock(node)\n                break",
     "                break"),
    ("admission matches every token", "m, blocks, node = self.match_prefix(list(toks)[:-1])",
     "m, blocks, node = self.match_prefix(list(toks))"),
    ("finish forgets to unlock", "            self.unlock(node)\n            self.pool.free(seq)",
     "            self.pool.free(seq)"),
    ("partial blocks cached", "for i in range(len(tokens) // bs)]", "for i in range(-(-len(tokens) // bs))]"),
]

POOL_MUTANTS = [
    ("release frees one reference early", "self._ref[block] -= 1\n        if self._ref[block] == 0:",
     "self._ref[block] -= 1\n        if self._ref[block] <= 1:"),
    ("prefix blocks take no reference", "for b in prefix_blocks:\n            self._ref[b] += 1",
     "for b in prefix_blocks:\n            self._ref[b] += 0"),
]

_RADIX_IMPORTS = [("from .pool import RefPool", "from oracle.pool import RefPool")]


@pytest.mark.parametrize("label,old,new", RADIX_MUTANTS, ids=[m[0] for m in RADIX_MUTANTS])
def test_radix_mutant_is_caught(label, old, new):
    mod = _load("radix.py", old, new, _RADIX_IMPORTS)
    with pytest.raises(AssertionError):
        rc.run_radix_pins(mod.RadixCache, RefPool)


@pytest.mark.parametrize("label,old,new", POOL_MUTANTS, ids=[m[0] for m in POOL_MUTANTS])
def test_pool_prefix_mutant_is_caught(label, old, new):
    pool = _load("pool.py", old, new, [])
    with pytest.raises(AssertionError):
        rc.run_radix_pins(RadixCache, pool.RefPool)


def test_unmutated_copies_pass():
    mod = _load("radix.py", "import math", "import math", _RADIX_IMPORTS)
    pool = _load("pool.py", "from collections import deque", "from collections import deque", [])
    rc.run_radix_pins(mod.RadixCache, pool.RefPool)

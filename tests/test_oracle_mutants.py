"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pin suite catches every one of them."""

import importlib.util
import os
import sys
import types

import pytest

import oracle_checks as oc

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _load_mutant(module_file, old, new):
    src = open(os.path.join(ORACLE_DIR, module_file)).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant_" + module_file.replace(".", "_"))
    exec(compile(src, module_file, "exec"), mod.__dict__)
    return mod


ATTENTION_MUTANTS = [
    ("wrong GQA head mapping", "kh = h // group", "kh = h % Hkv"),
    ("dropped softmax scale", "s = scale * (K[:, kh, :] @ qb[h])", "s = (K[:, kh, :] @ qb[h])"),
    ("K and V swapped", "out[i, h] = (p @ V[:, kh, :]) / p.sum()", "out[i, h] = (p @ K[:, kh, :]) / p.sum()"),
    ("missing normalisation", "out[i, h] = (p @ V[:, kh, :]) / p.sum()", "out[i, h] = (p @ V[:, kh, :])"),
    ("sign of the max shift", "p = np.exp(s - s.max())", "p = np.exp(s.max() - s)"),
    ("off-by-one token count", "reshape(nb * block_size, Hkv, d)[:n]\n        V", "reshape(nb * block_size, Hkv, d)[1:n + 1]\n        V"),
    ("bf16 decoded with a wrong shift", "wide = x.astype(np.uint32) << np.uint32(16)", "wide = x.astype(np.uint32) << np.uint32(15)"),
    ("blocks gathered in reverse", "ids = block_tables[b, :nb].astype(np.int64)", "ids = block_tables[b, :nb][::-1].astype(np.int64)"),
    ("wrong query row", "qb = decode_bits(q[b], dtype)", "qb = decode_bits(q[(b + 1) % B], dtype)"),
]


@pytest.mark.parametrize("label,old,new", ATTENTION_MUTANTS, ids=[m[0] for m in ATTENTION_MUTANTS])
def test_attention_mutant_is_caught(label, old, new):
    mod = _load_mutant("attention.py", old, new)
    with pytest.raises(AssertionError):
        oc.run_attention_pins(mod.ref_decode, __import__("oracle").bruteforce_decode, mod.decode_bits)


POOL_MUTANTS = [
    ("copy-on-write of unshared blocks", "if self._ref[x] > 1:\n                    y", "if self._ref[x] >= 1:\n                    y"),
    ("copy-on-write never triggers", "if self._ref[x] > 1:\n                    y", "if self._ref[x] > 99:\n                    y"),
    ("fork forgets the count", "self._ref[b] += 1", "self._ref[b] += 0"),
    ("free leaks blocks", "if self._ref[b] == 0:\n                self._free.append(b)", "if self._ref[b] == -1:\n                self._free.append(b)"),
    ("copy moves one row too few", "k[dst, :rows] = k[src, :rows]", "k[dst, :rows - 1] = k[src, :rows - 1]"),
    ("slot row off by one", "slots.append(table[j] * self.block_size + off)", "slots.append(table[j] * self.block_size + (off + 1) % self.block_size)"),
    ("alloc rounds down", "need = -(-int(num_tokens) // self.block_size)", "need = int(num_tokens) // self.block_size"),
    ("no capacity pre-check", "if need > len(self._free):\n            raise MemoryError(f\"OOM: append", "if False:\n            raise MemoryError(f\"OOM: append"),
]


@pytest.mark.parametrize("label,old,new", POOL_MUTANTS, ids=[m[0] for m in POOL_MUTANTS])
def test_pool_mutant_is_caught(label, old, new):
    mod = _load_mutant("pool.py", old, new)
    with pytest.raises(AssertionError):
        oc.run_pool_pins(mod.RefPool, mod.apply_append)


def test_unmutated_copies_pass():
    att = _load_mutant("attention.py", "import math", "import math")
    oc.run_attention_pins(att.ref_decode, att.bruteforce_decode, att.decode_bits)
    pool = _load_mutant("pool.py", "import numpy as np", "import numpy as np")
    oc.run_pool_pins(pool.RefPool, pool.apply_append)

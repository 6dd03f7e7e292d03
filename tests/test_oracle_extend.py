"""The extend (multi-token) oracle against its pins, and planted mistakes in copies of it."""

import os
import types

import pytest

import oracle
import oracle_checks as oc

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def test_extend_oracle_pins():
    oc.run_extend_pins(oracle.ref_extend, oracle.ref_decode, oracle.bruteforce_decode)


def _load_extend(old, new):
    src = open(os.path.join(ORACLE_DIR, "extend.py")).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new, 1).replace("from .attention import decode_bits", "from oracle.attention import decode_bits")
    mod = types.ModuleType("oracle_mutant_extend")
    exec(compile(src, "extend.py", "exec"), mod.__dict__)
    return mod


EXTEND_MUTANTS = [
    ("query sees one token too few",
     "s = scale * (K[: p + 1, kh, :] @ qr[h])\n            w = np.exp(s - s.max())\n            out[j, h] = (w @ V[: p + 1, kh, :])",
     "s = scale * (K[: max(p, 1), kh, :] @ qr[h])\n            w = np.exp(s - s.max())\n            out[j, h] = (w @ V[: max(p, 1), kh, :])"),
    ("query sees one token too many", "out.extend((b, n - ql + i) for i in range(ql))",
     "out.extend((b, n - ql + i + 1) for i in range(ql))"),
    ("no causal mask",
     "s = scale * (K[: p + 1, kh, :] @ qr[h])\n            w = np.exp(s - s.max())\n            out[j, h] = (w @ V[: p + 1, kh, :])",
     "s = scale * (K[:, kh, :] @ qr[h])\n            w = np.exp(s - s.max())\n            out[j, h] = (w @ V[:, kh, :])"),
    ("positions counted from 0", "out.extend((b, n - ql + i) for i in range(ql))", "out.extend((b, i) for i in range(ql))"),
    ("query tokens reversed", "out.extend((b, n - ql + i) for i in range(ql))", "out.extend((b, n - 1 - i) for i in range(ql))"),
    ("values not truncated", "out[j, h] = (w @ V[: p + 1, kh, :]) / w.sum()", "out[j, h] = (w @ V[-(p + 1):, kh, :]) / w.sum()"),
]


@pytest.mark.parametrize("label,old,new", EXTEND_MUTANTS, ids=[m[0] for m in EXTEND_MUTANTS])
def test_extend_mutant_is_caught(label, old, new):
    mod = _load_extend(old, new)
    with pytest.raises(AssertionError):
        oc.run_extend_pins(mod.ref_extend, oracle.ref_decode, oracle.bruteforce_decode)


def test_unmutated_extend_copy_passes():
    mod = _load_extend("import numpy as np", "import numpy as np")
    oc.run_extend_pins(mod.ref_extend, oracle.ref_decode, oracle.bruteforce_decode)

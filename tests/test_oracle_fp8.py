"""FP8 (E4M3) page format of the oracle against the format's definition, brute force and exact
special cases, with planted mistakes in copies of it."""

import os
import types

import numpy as np
import pytest

import oracle
import oracle_checks as oc

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def run_fp8_pins(fp8):
    # format definition (OCP E4M3, "fn" variant): exact special values
    v = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x3C] == 1.5 and v[0x40] == 2.0 and v[0x77] == 240.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and v[0x80] == 0 and np.signbit(v[0x80])
    assert np.all(np.diff(v[:0x7F]) > 0) and np.array_equal(v[0x80:0xFF], -v[:0x7F])
    # encoder: round trip, nearest value by brute force, ties to the even code
    codes = np.concatenate([np.arange(0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    assert np.array_equal(fp8.e4m3_encode(v[codes]), codes)
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.uniform(-0.05, 0.05, 3000),
                        (v[1:0x7E] + v[2:0x7F]) / 2])  # every midpoint: a tie
    got = fp8.e4m3_decode(fp8.e4m3_encode(x))
    finite = v[codes]
    dist = np.abs(finite[None, :] - x[:, None])
    best = dist.min(axis=1)
    assert np.array_equal(np.abs(got - x), best)
    mids = (v[1:0x7E] + v[2:0x7F]) / 2
    mid_codes = fp8.e4m3_encode(mids)
    assert np.all(mid_codes % 2 == 0)
    # scale exponent: the smallest k with amax / 2^k <= 448, by brute force over k
    amax = np.concatenate([448.0 * 2.0 ** np.arange(-20, 20), rng.uniform(0, 1, 500) * 10.0 **
                           rng.integers(-8, 8, 500), [449.0, 447.9, 1e-30]])
    k = fp8.pow2_scale_exponent(amax)
    for a, kk in zip(amax, k):
        ok = [j for j in range(-126, 128) if a / 2.0 ** j <= 448]
        assert kk == ok[0], (a, kk)
    assert fp8.pow2_scale_exponent(0.0) == 0
    # quantization error bound: half a unit in the last place of the 3-bit mantissa
    xs = rng.standard_normal((200, 64)) * 10.0 ** rng.integers(-3, 3, (200, 1))
    c, s = fp8.quantize_heads(xs)
    err = np.abs(fp8.dequantize_heads(c, s) - xs)
    assert np.all(err <= np.maximum(np.abs(xs) * 2.0 ** -4, s[:, None] * 2.0 ** -10))
    # page layout: scales are [block, head, row]; values exactly on the scaled grid dequantize to themselves
    nblk, bs, hkv, d = 3, 4, 2, 4
    codes_p = rng.integers(0, 0x7F, (nblk, bs, hkv, d)).astype(np.uint8)
    codes_p[..., 0] = 0x7E  # each head vector's amax is 448 * scale
    scales_p = 2.0 ** rng.integers(-6, 6, (nblk, hkv, bs))
    deq = fp8.dequantize_pages(codes_p, scales_p)
    for b in range(nblk):
        for r in range(bs):
            for h in range(hkv):
                assert np.array_equal(deq[b, r, h], v[codes_p[b, r, h]] * scales_p[b, h, r])
    # re-quantizing dequantized values gives the same codes and scales back
    c2, s2 = fp8.quantize_heads(deq)
    assert np.array_equal(c2, codes_p) and np.array_equal(s2, np.transpose(scales_p, (0, 2, 1)))


def run_fp8_decode_pin(fp8):
    """FP8 pages holding values that are exactly bf16 numbers decode like those bf16 numbers."""
    rng = np.random.default_rng(8)
    lens = [7, 13, 1]
    q, _, _, bt, sl = oc.random_paged_case(rng, 3, 4, 2, 8, 4, lens, "bf16")
    nblk = int(bt.max()) + 2
    kc = rng.integers(0, 0x7F, (nblk, 4, 2, 8)).astype(np.uint8) | (rng.integers(0, 2, (nblk, 4, 2, 8)) << 7).astype(np.uint8)
    vc = rng.integers(0, 0x7F, (nblk, 4, 2, 8)).astype(np.uint8)
    ks = 2.0 ** rng.integers(-4, 3, (nblk, 2, 4)).astype(np.float32)
    vs = 2.0 ** rng.integers(-4, 3, (nblk, 2, 4)).astype(np.float32)
    kd, vd = fp8.dequantize_pages(kc, ks), fp8.dequantize_pages(vc, vs)
    kb, vb = oc.bf16_bits(kd), oc.bf16_bits(vd)  # exact: at most 4 significant bits
    assert np.array_equal(oracle.decode_bits(kb, "bf16"), kd)
    a = fp8.ref_decode_fp8(q, kc, vc, ks, vs, bt, sl, 0.7, "bf16")
    b = oracle.ref_decode(q, kb, vb, bt, sl, 0.7, "bf16")
    assert np.array_equal(a, b)


def run_fp8_extend_pin(fp8):
    """FP8 extend over bf16-exact values equals the extend oracle on those bf16 pages bit
    for bit, and one query token per row equals the FP8 decode oracle."""
    rng = np.random.default_rng(9)
    lens = [9, 14, 5]
    q_lens = [3, 1, 5]
    _, _, _, bt, sl = oc.random_paged_case(rng, 3, 4, 2, 8, 4, lens, "bf16")
    nblk = int(bt.max()) + 2
    kc = rng.integers(0, 0x7F, (nblk, 4, 2, 8)).astype(np.uint8) | (rng.integers(0, 2, (nblk, 4, 2, 8)) << 7).astype(np.uint8)
    vc = rng.integers(0, 0x7F, (nblk, 4, 2, 8)).astype(np.uint8)
    ks = 2.0 ** rng.integers(-4, 3, (nblk, 2, 4)).astype(np.float32)
    vs = 2.0 ** rng.integers(-4, 3, (nblk, 2, 4)).astype(np.float32)
    kb, vb = oc.bf16_bits(fp8.dequantize_pages(kc, ks)), oc.bf16_bits(fp8.dequantize_pages(vc, vs))
    q = oc.bf16_bits(rng.standard_normal((sum(q_lens), 4, 8)))
    a = fp8.ref_extend_fp8(q, kc, vc, ks, vs, bt, sl, q_lens, 0.6, "bf16")
    b = oracle.ref_extend(q, kb, vb, bt, sl, q_lens, 0.6, "bf16")
    assert np.array_equal(a, b)
    last = np.cumsum(q_lens) - 1  # each row's last query token sits at its last position
    d = fp8.ref_decode_fp8(q[last], kc, vc, ks, vs, bt, sl, 0.6, "bf16")
    assert np.allclose(a[last], d, rtol=0, atol=1e-12)


def test_fp8_extend_pin():
    run_fp8_extend_pin(oracle.fp8)


def test_fp8_format_pins():
    run_fp8_pins(oracle.fp8)


def test_fp8_decode_pin():
    run_fp8_decode_pin(oracle.fp8)


def run_fp8_append_pin(fp8):
    """A planned append onto FP8 pages: the copy-on-write moves rows [0, rows) of the
    source's K and V codes and scales, the token's K and V head vectors land quantized
    in its slot (each from its own input), and nothing else changes."""
    from oracle.attention import decode_bits

    rng = np.random.default_rng(2)
    nblk, bs, hkv, d = 6, 4, 2, 8
    kc = rng.integers(0, 256, (nblk, bs, hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (nblk, bs, hkv, d)).astype(np.uint8)
    ks = rng.random((nblk, hkv, bs)).astype(np.float32)
    vs = rng.random((nblk, hkv, bs)).astype(np.float32)
    kn = oc.bf16_bits(rng.standard_normal((2, hkv, d)) * 3)
    vn = oc.bf16_bits(rng.standard_normal((2, hkv, d)) * 0.01)
    slots, cows = [4 * 3 + 2, -1], [(1, 3, 2)]
    k2, v2, ks2, vs2 = fp8.apply_append_fp8(kc, vc, ks, vs, slots, cows, kn, vn, "bf16")
    # copy-on-write: rows 0, 1 of block 1 into block 3, codes and scales of K and of V
    assert np.array_equal(k2[3, :2], kc[1, :2]) and np.array_equal(ks2[3, :, :2], ks[1, :, :2])
    assert np.array_equal(v2[3, :2], vc[1, :2]) and np.array_equal(vs2[3, :, :2], vs[1, :, :2])
    # the token in slot (3, 2): K from k_new, V from v_new, with their scales
    kq, ksq = fp8.quantize_heads(decode_bits(kn[0], "bf16"))
    vq, vsq = fp8.quantize_heads(decode_bits(vn[0], "bf16"))
    assert not np.array_equal(kq, vq) and not np.array_equal(ksq, vsq)  # the inputs tell K and V apart
    assert np.array_equal(k2[3, 2], kq) and np.array_equal(ks2[3, :, 2], ksq)
    assert np.array_equal(v2[3, 2], vq) and np.array_equal(vs2[3, :, 2], vsq)
    # everything else unchanged: other blocks, and row 3 of block 3 (slot -1 writes nothing)
    untouched = [b for b in range(nblk) if b != 3]
    for new_arr, old_arr in ((k2, kc), (v2, vc)):
        assert np.array_equal(new_arr[untouched], old_arr[untouched])
        assert np.array_equal(new_arr[3, 3], old_arr[3, 3])
    for new_arr, old_arr in ((ks2, ks), (vs2, vs)):
        assert np.array_equal(new_arr[untouched], old_arr[untouched])
        assert np.array_equal(new_arr[3, :, 3], old_arr[3, :, 3])


def test_fp8_append_copies_and_quantizes():
    run_fp8_append_pin(oracle.fp8)


def _load_fp8(old, new):
    src = open(os.path.join(ORACLE_DIR, "fp8.py")).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    src = src.replace(old, new, 1).replace("from .attention import", "from oracle.attention import")
    src = src.replace("from .extend import", "from oracle.extend import")
    mod = types.ModuleType("oracle_mutant_fp8")
    exec(compile(src, "fp8.py", "exec"), mod.__dict__)
    return mod


FP8_MUTANTS = [
    ("subnormals off by a factor 2", "m * 2.0 ** -9", "m * 2.0 ** -10"),
    ("exponent bias 8", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("ties away from zero", "np.where(lo % 2 == 0, lo, hi)", "hi"),
    ("scale one power too large", "k = np.where(m <= 0.875, e - 9, e - 8)", "k = np.where(m <= 0.875, e - 8, e - 7)"),
    ("scale threshold at 1.0", "k = np.where(m <= 0.875, e - 9, e - 8)", "k = np.where(m < 0.5, e - 9, e - 8)"),
    ("scales indexed [block, row, head]", "sc = np.transpose(np.asarray(scales, dtype=np.float64), (0, 2, 1))",
     "sc = np.asarray(scales, dtype=np.float64).reshape(np.asarray(scales).shape[0], -1, np.asarray(scales).shape[1])"),
    ("sign dropped", "return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)",
     "return code.astype(np.uint8)"),
    ("V quantized from k_new", "vq, vsc = quantize_heads(decode_bits(np.asarray(v_new), dtype))",
     "vq, vsc = quantize_heads(decode_bits(np.asarray(k_new), dtype))"),
    ("V scale not written", "ks[blk, :, row], vs[blk, :, row] = ksc[i], vsc[i]", "ks[blk, :, row] = ksc[i]"),
    ("V codes not copied on write", "        vc[dst, :rows] = vc[src, :rows]\n", ""),
    ("V scales not copied on write", "        vs[dst, :, :rows] = vs[src, :, :rows]\n", ""),
]


@pytest.mark.parametrize("label,old,new", FP8_MUTANTS, ids=[m[0] for m in FP8_MUTANTS])
def test_fp8_mutant_is_caught(label, old, new):
    mod = _load_fp8(old, new)
    with pytest.raises(AssertionError):
        run_fp8_pins(mod)
        run_fp8_decode_pin(mod)
        run_fp8_append_pin(mod)


def test_unmutated_fp8_copy_passes():
    mod = _load_fp8("import numpy as np", "import numpy as np")
    run_fp8_pins(mod)
    run_fp8_decode_pin(mod)
    run_fp8_append_pin(mod)

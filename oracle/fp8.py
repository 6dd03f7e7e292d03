"""FP8 (E4M3) KV pages with per-(token, head) power-of-two scales (oracle; test infrastructure only).

"The Reasoning Engine Meltdown" names FP8 among the KV-cache compressions that
make deep search trees fit (§3 and its conclusion, FP4/FP8 quantization); the
pages fix no format, scale granularity or rounding.  Readings:

* Format: OCP 8-bit floating point E4M3 ("fn": no infinities, one NaN pattern
  per sign, largest finite 448, subnormals down to 2^-9).
* Scale: one per token and KV head (so appending a token never re-quantizes the
  rest of its block), a power of two 2^k with k the smallest integer such that
  max |x| / 2^k <= 448, kept inside the normal fp32 exponents [-126, 127];
  x / 2^k is then exact and is rounded to the nearest E4M3 value, ties to even.
  An all-zero vector gets k = 0.
* Layout: codes [num_blocks, block_size, Hkv, d] uint8 (the 16-bit page layout
  with one byte per element); scales [num_blocks, Hkv, block_size] float32.
* Dequantized value: code value * 2^k, exact in fp32 and fp64.

Everything here is plain numpy, written from the format's definition.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes):
    """float64 values of E4M3 codes (uint8); NaN for the NaN patterns."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_POS_CODES = np.arange(0x7F, dtype=np.uint8)  # 0x00 .. 0x7E: every finite non-negative value, increasing
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x):
    """E4M3 codes of finite values with |x| <= 448: nearest value, ties to the even code."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode takes finite values with |x| <= 448")
    a = np.abs(x)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALUES) - 1)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    code = _POS_CODES[pick].astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)


def pow2_scale_exponent(amax):
    """Smallest integer k with amax / 2^k <= 448 (k = 0 for amax == 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    m, e = np.frexp(amax)  # amax = m * 2^e, m in [0.5, 1)
    k = np.where(m <= 0.875, e - 9, e - 8)
    k = np.clip(k, -126, 127)
    return np.where(amax == 0, 0, k).astype(np.int64)


def quantize_heads(x):
    """x [..., d] float -> (codes uint8 [..., d], scales float32 [...]) per head vector."""
    x = np.asarray(x, dtype=np.float64)
    k = pow2_scale_exponent(np.max(np.abs(x), axis=-1))
    scale = np.exp2(k.astype(np.float64))
    codes = e4m3_encode(x / scale[..., None])
    return codes, scale.astype(np.float32)


def dequantize_heads(codes, scales):
    """codes [..., d] uint8, scales [...] -> float64 values."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def apply_append_fp8(k_codes, v_codes, k_scales, v_scales, slots, cows, k_new, v_new, dtype):
    """Planned append onto FP8 pages (returns new arrays): copy-on-write copies rows
    [0, rows) of codes and scales, then every token's K / V head vectors (16-bit
    bit patterns of ``dtype``) are quantized into its slot."""
    from .attention import decode_bits

    kc, vc = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    ks, vs = np.array(k_scales, copy=True), np.array(v_scales, copy=True)
    block_size = kc.shape[1]
    for src, dst, rows in cows:
        kc[dst, :rows] = kc[src, :rows]
        vc[dst, :rows] = vc[src, :rows]
        ks[dst, :, :rows] = ks[src, :, :rows]
        vs[dst, :, :rows] = vs[src, :, :rows]
    kq, ksc = quantize_heads(decode_bits(np.asarray(k_new), dtype))
    vq, vsc = quantize_heads(decode_bits(np.asarray(v_new), dtype))
    for i, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        blk, row = divmod(slot, block_size)
        kc[blk, row], vc[blk, row] = kq[i], vq[i]
        ks[blk, :, row], vs[blk, :, row] = ksc[i], vsc[i]
    return kc, vc, ks, vs


def dequantize_pages(codes, scales):
    """FP8 pages [num_blocks, block_size, Hkv, d] with scales [num_blocks, Hkv, block_size]
    -> float64 pages of the same shape."""
    sc = np.transpose(np.asarray(scales, dtype=np.float64), (0, 2, 1))  # [num_blocks, block_size, Hkv]
    return e4m3_decode(codes) * sc[..., None]


def ref_decode_fp8(q, k_codes, v_codes, k_scales, v_scales, block_tables, seq_lens, scale, q_dtype):
    """Decode attention over FP8 pages: the plain definition on the dequantized values
    (q given as 16-bit bit patterns of ``q_dtype``)."""
    from .attention import decode_bits, ref_decode

    return ref_decode(decode_bits(q, q_dtype), dequantize_pages(k_codes, k_scales),
                      dequantize_pages(v_codes, v_scales), block_tables, seq_lens, scale, "f64")


def ref_extend_fp8(q, k_codes, v_codes, k_scales, v_scales, block_tables, seq_lens, q_lens, scale, q_dtype,
                   query_rows=None):
    """Multi-token (extend) attention over FP8 pages: the extend oracle on the
    dequantized values (q given as 16-bit bit patterns of ``q_dtype``)."""
    from .attention import decode_bits
    from .extend import ref_extend

    return ref_extend(decode_bits(q, q_dtype), dequantize_pages(k_codes, k_scales), dequantize_pages(v_codes, v_scales),
                      block_tables, seq_lens, q_lens, scale, "f64", query_rows)

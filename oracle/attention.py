"""Single-token decode attention over a paged KV cache (oracle; test infrastructure only).

What is computed, and where the pages define it:

* "The Reasoning Engine Meltdown", §2.1: Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V
  (the formula is garbled in the extracted text; this is its standard reading),
  and the decode step: the query of step t+1 attends to the cached keys and
  values K_{1:t}, V_{1:t}.
* "Dismantling the Memory Wall", section "PagedAttention: The Virtual Memory
  Analogy for GPUs": the cache is cut into fixed 16-token blocks scattered in
  memory, and a per-sequence block table maps logical block
  ``token_idx // block_size`` to a physical block.

Readings where the pages are silent (each listed in the design notes):

* The softmax scale is an explicit argument; callers pass 1/sqrt(d).
* Grouped-query attention: query head h reads KV head h // group, with
  group = Hq // Hkv (consecutive query heads share a KV head, the same as
  ``repeat_interleave`` of the KV heads).
* A row attends to exactly ``seq_lens[b]`` tokens of its table; a row with
  ``seq_lens[b] == 0`` has output 0.
* Table entries past ceil(len / block_size) are never read.

Layouts: q [B, Hq, d]; k_pages, v_pages [num_blocks, block_size, Hkv, d]; all
three as raw fp16 or bf16 bit patterns (uint16) or as float arrays.
block_tables [B, max_blocks] int; seq_lens [B] int.  Output: float64 [B, Hq, d].
"""

import math
import struct

import numpy as np


def decode_bits(x, dtype: str) -> np.ndarray:
    """Turn raw 16-bit patterns into float64 values.

    ``dtype`` is "f16" (IEEE binary16) or "bf16" (the upper half of an IEEE
    binary32).  "f32"/"f64" pass float arrays through unchanged (used by the
    closed-form tests, which build exact values directly).
    """
    x = np.asarray(x)
    if dtype == "f16":
        return x.astype(np.uint16, copy=False).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = x.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f64"):
        return x.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _check_shapes(q, k_pages, v_pages, block_tables, seq_lens):
    if q.ndim != 3 or k_pages.ndim != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("q must be [B,Hq,d]; k/v pages [num_blocks, block_size, Hkv, d] of equal shape")
    B, Hq, d = q.shape
    num_blocks, block_size, Hkv, dk = k_pages.shape
    if dk != d:
        raise ValueError("head_dim of q and pages differ")
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if block_tables.ndim != 2 or block_tables.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_tables must be [B, max_blocks] and seq_lens [B]")
    return B, Hq, d, num_blocks, block_size, Hkv


def ref_decode_rows(q, k_pages, v_pages, block_tables, seq_lens, scale, dtype, rows=None):
    """Oracle output for the decode rows in ``rows`` (all rows if None).

    For each row b: gather its ceil(n/block_size) blocks through the block table
    into contiguous K and V of n tokens, then for every query head h compute
    softmax(scale * K_h q_h) V_h in fp64, with K_h, V_h the keys and values of
    KV head h // group.  Returns an array [len(rows), Hq, d].
    """
    q = np.asarray(q)
    k_pages = np.asarray(k_pages)
    v_pages = np.asarray(v_pages)
    block_tables = np.asarray(block_tables)
    seq_lens = np.asarray(seq_lens)
    B, Hq, d, num_blocks, block_size, Hkv = _check_shapes(q, k_pages, v_pages, block_tables, seq_lens)
    group = Hq // Hkv
    rows = range(B) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(rows), Hq, d), dtype=np.float64)
    for i, b in enumerate(rows):
        n = int(seq_lens[b])
        if n < 0:
            raise ValueError(f"seq_lens[{b}] = {n} is negative")
        if n == 0:
            continue  # empty row: output stays 0
        nb = -(-n // block_size)  # blocks that hold tokens 0..n-1
        if nb > block_tables.shape[1]:
            raise IndexError(f"row {b}: {n} tokens need {nb} blocks, table has {block_tables.shape[1]}")
        ids = block_tables[b, :nb].astype(np.int64)
        if (ids < 0).any() or (ids >= num_blocks).any():
            raise IndexError(f"row {b}: block id out of range")
        # token t lives in physical block ids[t // block_size], row t % block_size
        K = decode_bits(k_pages[ids], dtype).reshape(nb * block_size, Hkv, d)[:n]
        V = decode_bits(v_pages[ids], dtype).reshape(nb * block_size, Hkv, d)[:n]
        qb = decode_bits(q[b], dtype)
        for h in range(Hq):
            kh = h // group
            s = scale * (K[:, kh, :] @ qb[h])
            p = np.exp(s - s.max())
            out[i, h] = (p @ V[:, kh, :]) / p.sum()
    return out


def ref_decode(q, k_pages, v_pages, block_tables, seq_lens, scale, dtype):
    """Oracle output o[B, Hq, d] (float64) for every decode row."""
    return ref_decode_rows(q, k_pages, v_pages, block_tables, seq_lens, scale, dtype, rows=None)


# ---------------------------------------------------------------------------
# A second, deliberately different implementation for tiny inputs: pure Python,
# one token at a time through the block table (no gather, no numpy algebra, its
# own bit decoding).  It exists only to pin ``ref_decode``.


def _scalar_from_bits(bits: int, dtype: str) -> float:
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    raise ValueError(dtype)


def bruteforce_decode(q, k_pages, v_pages, block_tables, seq_lens, scale, dtype, max_work=2_000_000):
    """Token-by-token reference for tiny inputs; returns nested Python lists [B][Hq][d]."""
    q = np.asarray(q)
    k_pages = np.asarray(k_pages)
    v_pages = np.asarray(v_pages)
    B, Hq, d = q.shape
    _, block_size, Hkv, _ = k_pages.shape
    group = Hq // Hkv
    if int(sum(int(n) for n in seq_lens)) * Hq * d > max_work:
        raise ValueError("bruteforce_decode is for tiny inputs only")

    def val(arr, idx):
        x = arr[idx]
        if dtype in ("f16", "bf16"):
            return _scalar_from_bits(int(x), dtype)
        return float(x)

    out = []
    for b in range(B):
        n = int(seq_lens[b])
        rows = []
        for h in range(Hq):
            if n == 0:
                rows.append([0.0] * d)
                continue
            kh = h // group
            qv = [val(q, (b, h, e)) for e in range(d)]
            scores = []
            where = []
            for t in range(n):
                phys = int(block_tables[b][t // block_size])  # logical block t // block_size
                r = t % block_size
                where.append((phys, r))
                scores.append(scale * math.fsum(qv[e] * val(k_pages, (phys, r, kh, e)) for e in range(d)))
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            denom = math.fsum(w)
            rows.append([
                math.fsum(w[t] * val(v_pages, (where[t][0], where[t][1], kh, e)) for t in range(n)) / denom
                for e in range(d)
            ])
        out.append(rows)
    return out

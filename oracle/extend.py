"""Multi-token (extend) attention over a paged KV cache (oracle; test infrastructure only).

Several new tokens of a sequence attend at once, each to the sequence's cache
up to and including its own position:

* "RKSC" (gist.science summary, §1): a verification pass scores a generated
  branch with one forward pass over its tokens, and the branches of one
  problem share their prefix.
* "Dismantling the Memory Wall", section "Chunked Prefill": a long prompt is
  processed in token slices; each slice's tokens attend to what was cached
  before them and, causally, to the slice itself.
* "The Reasoning Engine Meltdown", §2.1: the attention definition
  softmax(Q K^T / sqrt(d_k)) V, with the scale passed explicitly.

Reading (where the pages leave it open): row b's q_lens[b] query tokens are the
last q_lens[b] of its seq_lens[b] cached tokens (appended before the call);
query token i sits at position p = seq_lens[b] - q_lens[b] + i and attends to
tokens 0..p.  Query rows are packed in row order: rows of b start at
q_lens[0] + ... + q_lens[b-1].  GQA as in the decode oracle: query head h reads
KV head h // (Hq // Hkv).

Layouts: q [sum(q_lens), Hq, d]; pages [num_blocks, block_size, Hkv, d];
block_tables [B, max_blocks]; seq_lens, q_lens [B].  Output float64
[sum(q_lens), Hq, d].
"""

import numpy as np

from .attention import decode_bits


def extend_query_positions(seq_lens, q_lens):
    """(row, position) of every packed query row, in order."""
    out = []
    for b, (n, ql) in enumerate(zip(seq_lens, q_lens)):
        n, ql = int(n), int(ql)
        if ql < 0 or ql > n:
            raise ValueError(f"row {b}: q_lens {ql} outside [0, seq_lens {n}]")
        out.extend((b, n - ql + i) for i in range(ql))
    return out


def ref_extend(q, k_pages, v_pages, block_tables, seq_lens, q_lens, scale, dtype, query_rows=None):
    """Oracle output for the packed query rows in ``query_rows`` (all if None).

    For each query row (row b, position p): gather the row's blocks through its
    table into contiguous K and V, keep tokens 0..p, and compute
    softmax(scale * K_h q_h) V_h in fp64 for every query head h.
    """
    q = np.asarray(q)
    k_pages = np.asarray(k_pages)
    v_pages = np.asarray(v_pages)
    block_tables = np.asarray(block_tables)
    num_blocks, block_size, Hkv, d = k_pages.shape
    NQ, Hq, dq = q.shape
    if dq != d or Hq % Hkv != 0:
        raise ValueError("q must be [NQ, Hq, d] with Hq a multiple of Hkv")
    where = extend_query_positions(seq_lens, q_lens)
    if len(where) != NQ:
        raise ValueError(f"q has {NQ} rows, q_lens sum to {len(where)}")
    group = Hq // Hkv
    sel = range(NQ) if query_rows is None else [int(r) for r in query_rows]
    out = np.zeros((len(sel), Hq, d), dtype=np.float64)
    cache = {}
    for j, r in enumerate(sel):
        b, p = where[r]
        if b not in cache:
            n = int(seq_lens[b])
            nb = -(-n // block_size)
            ids = block_tables[b, :nb].astype(np.int64)
            if (ids < 0).any() or (ids >= num_blocks).any():
                raise IndexError(f"row {b}: block id out of range")
            K = decode_bits(k_pages[ids], dtype).reshape(nb * block_size, Hkv, d)[:n]
            V = decode_bits(v_pages[ids], dtype).reshape(nb * block_size, Hkv, d)[:n]
            cache = {b: (K, V)}  # one row at a time keeps memory bounded
        K, V = cache[b]
        qr = decode_bits(q[r], dtype)
        for h in range(Hq):
            kh = h // group
            s = scale * (K[: p + 1, kh, :] @ qr[h])
            w = np.exp(s - s.max())
            out[j, h] = (w @ V[: p + 1, kh, :]) / w.sum()
    return out

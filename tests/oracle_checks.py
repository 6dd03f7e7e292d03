"""Checks that pin the oracle to the source pages and to mathematics.

Each check takes the oracle functions as arguments so that the same suite can
be run against deliberately broken copies of the oracle (``test_oracle_mutants``):
a plausible mistake anywhere in the oracle must make at least one check fail.
"""

import math

import numpy as np

from conftest import read_golden


def f16_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def bf16_bits(x):
    """Round-to-nearest-even fp32 -> bf16 bit patterns (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def to_bits(x, dtype):
    return f16_bits(x) if dtype == "f16" else bf16_bits(x)


def random_paged_case(rng, B, Hq, Hkv, d, block_size, lens, dtype, nblk_extra=3):
    """Random q / pages / scattered block tables for explicit lengths."""
    need = [(-(-int(n) // block_size)) for n in lens]
    nblk = sum(need) + nblk_extra
    perm = rng.permutation(nblk)
    maxb = max(1, max(need))
    bt = np.full((B, maxb), -1, dtype=np.int32)
    pos = 0
    for b, nb in enumerate(need):
        bt[b, :nb] = perm[pos:pos + nb]
        pos += nb
    q = to_bits(rng.standard_normal((B, Hq, d)), dtype)
    k = to_bits(rng.standard_normal((nblk, block_size, Hkv, d)), dtype)
    v = to_bits(rng.standard_normal((nblk, block_size, Hkv, d)), dtype)
    return q, k, v, bt, np.asarray(lens, dtype=np.int32)


# ---------------------------------------------------------------------------
# KV-size formula


def check_kv_formula(kv_bytes):
    g = read_golden("kv_size_formula.txt")
    per_tok = kv_bytes(g["layers"], g["heads"], g["head_dim"], 1, g["elem_bytes"])
    assert per_tok == g["per_token_bytes"]
    assert round(per_tok / 1e6, 2) == g["per_token_mb_printed"]
    seq = kv_bytes(g["layers"], g["heads"], g["head_dim"], g["seq_tokens"], g["elem_bytes"])
    assert seq == g["seq_tokens"] * g["per_token_bytes"]
    assert round(seq / 1e9, 2) == g["seq_gb_printed"]
    layer = kv_bytes(1, g["layer_heads"], g["head_dim"], g["layer_batch"] * g["layer_tokens"], g["elem_bytes"])
    assert layer == 2 ** 32
    assert round(layer / 1e9, 1) == g["layer_gb_printed"]


# ---------------------------------------------------------------------------
# attention


def check_bruteforce(ref_decode, bruteforce_decode, seed=0):
    rng = np.random.default_rng(seed)
    cases = [
        # B, Hq, Hkv, d, block, lens, dtype
        (3, 2, 2, 4, 4, [5, 0, 9], "f16"),
        (3, 4, 2, 4, 4, [1, 12, 7], "bf16"),
        (2, 6, 3, 3, 4, [16, 13], "bf16"),
        (2, 4, 1, 4, 16, [17, 33], "f16"),
        (1, 2, 2, 8, 4, [40], "bf16"),
    ]
    for B, Hq, Hkv, d, bs, lens, dt in cases:
        q, k, v, bt, sl = random_paged_case(rng, B, Hq, Hkv, d, bs, lens, dt)
        scale = 1.0 / math.sqrt(d)
        o = ref_decode(q, k, v, bt, sl, scale, dt)
        ob = np.array(bruteforce_decode(q, k, v, bt, sl, scale, dt))
        assert o.shape == ob.shape == (B, Hq, d)
        assert np.max(np.abs(o - ob)) <= 1e-12, (B, Hq, Hkv, d, bs, lens, dt)


def check_closed_forms(ref_decode):
    rng = np.random.default_rng(11)
    bs, Hkv, d = 4, 2, 8
    # one token: softmax of one score is 1, so o = v_0 exactly
    q, k, v, bt, sl = random_paged_case(rng, 2, 4, Hkv, d, bs, [1, 1], "bf16")
    o = ref_decode(q, k, v, bt, sl, 0.7, "bf16")
    from oracle import decode_bits  # bit decoding is pinned separately below
    for b in range(2):
        for h in range(4):
            np.testing.assert_array_equal(o[b, h], decode_bits(v[bt[b, 0], 0, h // 2], "bf16"))
    # constant keys (and q = 0): every score equal -> o = mean of V over the attended tokens
    for case in ("const_k", "zero_q"):
        n = 11
        q, k, v, bt, sl = random_paged_case(rng, 1, 2, Hkv, d, bs, [n], "f16")
        if case == "const_k":
            k[:] = k[bt[0, 0], 0][None, None]
        else:
            q[:] = 0
        o = ref_decode(q, k, v, bt, sl, 1.0 / math.sqrt(d), "f16")
        V = decode_bits(v[bt[0, :3]], "f16").reshape(12, Hkv, d)[:n]
        for h in range(2):
            np.testing.assert_allclose(o[0, h], V[:, h].mean(axis=0), rtol=0, atol=1e-13)
    # a single dominant key: o ~= its value vector
    n = 9
    q, k, v, bt, sl = random_paged_case(rng, 1, 1, 1, d, bs, [n], "f16")
    qv = np.full(d, 1.0)
    q[0, 0] = f16_bits(qv)
    k[:] = f16_bits(np.zeros(d))
    hot = 6
    k[bt[0, hot // bs], hot % bs, 0] = f16_bits(np.full(d, 8.0))
    o = ref_decode(q, k, v, bt, sl, 1.0, "f16")
    # scores: 64 for the hot token, 0 elsewhere -> weight of others ~ 8 e^-64
    np.testing.assert_allclose(o[0, 0], decode_bits(v[bt[0, hot // bs], hot % bs, 0], "f16"), atol=1e-25)
    # empty row gives zeros
    q, k, v, bt, sl = random_paged_case(rng, 2, 2, 2, d, bs, [0, 3], "bf16")
    o = ref_decode(q, k, v, bt, sl, 1.0, "bf16")
    assert np.all(o[0] == 0)


def check_permutation_invariance(ref_decode, seed=5):
    rng = np.random.default_rng(seed)
    q, k, v, bt, sl = random_paged_case(rng, 3, 4, 2, 8, 4, [13, 4, 21], "bf16", nblk_extra=5)
    o1 = ref_decode(q, k, v, bt, sl, 0.35, "bf16")
    nblk = k.shape[0]
    pi = rng.permutation(nblk)  # block i moves to pi[i]
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[pi] = k
    v2[pi] = v
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1).astype(np.int32)
    o2 = ref_decode(q, k2, v2, bt2, sl, 0.35, "bf16")
    assert np.array_equal(o1, o2)
    # and the placement does matter: swapping a full block with the partly filled
    # last block changes which tokens the row attends to
    bt3 = bt.copy()
    bt3[0, 0], bt3[0, 3] = bt[0, 3], bt[0, 0]
    o3 = ref_decode(q, k, v, bt3, sl, 0.35, "bf16")
    assert not np.array_equal(o1[0], o3[0])


def check_gqa_equals_repeated_mha(ref_decode, seed=6):
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, bs = 6, 2, 4, 4
    g = Hq // Hkv
    q, k, v, bt, sl = random_paged_case(rng, 2, Hq, Hkv, d, bs, [7, 10], "f16")
    o = ref_decode(q, k, v, bt, sl, 0.5, "f16")
    k_rep = np.repeat(k, g, axis=2)  # repeat_interleave of the KV heads
    v_rep = np.repeat(v, g, axis=2)
    o_mha = ref_decode(q, k_rep, v_rep, bt, sl, 0.5, "f16")
    assert np.array_equal(o, o_mha)


def check_convex_hull(ref_decode, seed=7):
    rng = np.random.default_rng(seed)
    from oracle import decode_bits
    q, k, v, bt, sl = random_paged_case(rng, 3, 2, 1, 8, 4, [5, 17, 30], "bf16")
    o = ref_decode(q, k, v, bt, sl, 2.0, "bf16")
    for b in range(3):
        n = sl[b]
        nb = -(-n // 4)
        V = decode_bits(v[bt[b, :nb]], "bf16").reshape(nb * 4, 1, 8)[:n, 0]
        assert np.all(o[b] >= V.min(axis=0) - 1e-12) and np.all(o[b] <= V.max(axis=0) + 1e-12)


def check_sdpa(ref_decode, seed=8):
    import torch
    from oracle import decode_bits

    rng = np.random.default_rng(seed)
    Hq, Hkv, d, bs = 4, 2, 16, 16
    q, k, v, bt, sl = random_paged_case(rng, 2, Hq, Hkv, d, bs, [37, 64], "bf16")
    o = ref_decode(q, k, v, bt, sl, 0.25, "bf16")
    for b in range(2):
        n = int(sl[b])
        nb = -(-n // bs)
        K = torch.from_numpy(decode_bits(k[bt[b, :nb]], "bf16").reshape(nb * bs, Hkv, d)[:n])
        V = torch.from_numpy(decode_bits(v[bt[b, :nb]], "bf16").reshape(nb * bs, Hkv, d)[:n])
        Kr = K.repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
        Vr = V.repeat_interleave(Hq // Hkv, dim=1).permute(1, 0, 2).unsqueeze(0).contiguous()
        Q = torch.from_numpy(decode_bits(q[b], "bf16")).unsqueeze(0).unsqueeze(2)  # [1,Hq,1,d]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kr, Vr, scale=0.25)[0, :, 0].numpy()
        np.testing.assert_allclose(o[b], ref, rtol=0, atol=1e-12)


def check_decode_bits(decode_bits):
    # exact values from the IEEE formats
    assert decode_bits(np.array([0x3C00], np.uint16), "f16")[0] == 1.0
    assert decode_bits(np.array([0xC000], np.uint16), "f16")[0] == -2.0
    assert decode_bits(np.array([0x0001], np.uint16), "f16")[0] == 2.0 ** -24
    assert decode_bits(np.array([0x3F80], np.uint16), "bf16")[0] == 1.0
    assert decode_bits(np.array([0xC040], np.uint16), "bf16")[0] == -3.0
    assert decode_bits(np.array([0x3F81], np.uint16), "bf16")[0] == 1.0 + 2.0 ** -7


def run_attention_pins(ref_decode, bruteforce_decode, decode_bits):
    check_decode_bits(decode_bits)
    check_bruteforce(ref_decode, bruteforce_decode)
    check_closed_forms(ref_decode)
    check_permutation_invariance(ref_decode)
    check_gqa_equals_repeated_mha(ref_decode)
    check_convex_hull(ref_decode)
    check_sdpa(ref_decode)


# ---------------------------------------------------------------------------
# block pool


def check_worked_example(RefPool):
    g = read_golden("fork_refcount_example.txt")
    bs = g["block_size"]
    pool = RefPool(8, bs)
    root = pool.alloc("R", g["root_tokens"])
    assert len(root) == 1
    pool.fork("R", "A")
    pool.fork("R", "B")
    pool.free("R")
    assert pool.refcount(root[0]) == g["refcount_root_block"]
    for s in ("A", "B"):
        while pool.length(s) < g["branch_tokens"]:
            slots, cows = pool.plan_append([s])
            assert cows == []  # the append at token 16 opens a new block: nothing to copy
    ta, tb = pool.table("A"), pool.table("B")
    assert len(ta) == len(tb) == g["blocks_per_branch"]
    assert ta[0] == tb[0] == root[0]
    assert ta[1] != tb[1]
    assert pool.refcount(ta[1]) == g["refcount_branch_a_block"]
    assert pool.refcount(tb[1]) == g["refcount_branch_b_block"]
    assert pool.refcount(root[0]) == g["refcount_root_block"]


def expect_error(exc, fn, *args):
    """Pin: fn(*args) raises exc.  Any other outcome (no error, or another exception
    type, e.g. a crash halfway through a batch) fails the pin as an assertion."""
    try:
        fn(*args)
    except exc:
        return
    except Exception as e:  # noqa: BLE001 - a different error is a failed pin
        raise AssertionError(f"expected {exc.__name__}, got {type(e).__name__}: {e}") from e
    raise AssertionError(f"expected {exc.__name__}")


def check_error_conventions(RefPool):
    pool = RefPool(4, 4)
    pool.alloc("x", 9)  # 3 blocks
    before = (pool.free_list(), pool.table("x"))
    expect_error(MemoryError, pool.alloc, "y", 5)  # needs 2, 1 free
    assert (pool.free_list(), pool.table("x")) == before and "y" not in pool
    expect_error(KeyError, pool.fork, "nope", "z")
    pool.free("never-allocated")  # no-op
    assert pool.free_list() == before[0]
    # an append batch that cannot fit changes nothing
    pool.fork("x", "x2")
    pool.fork("x", "x3")  # tail block (1 of 4 rows used) shared by three
    snap = (pool.free_list(), pool.table("x"), pool.table("x2"), pool.table("x3"),
            [pool.refcount(b) for b in range(4)], pool.length("x"))
    expect_error(MemoryError, pool.plan_append, ["x", "x2", "x3"])  # two copies needed, one block free
    assert snap == (pool.free_list(), pool.table("x"), pool.table("x2"), pool.table("x3"),
                    [pool.refcount(b) for b in range(4)], pool.length("x"))


def check_pool_against_unpaged_model(RefPool, apply_append, seed=0, n_ops=400):
    """Random alloc/fork/append/free on a tiny pool against a plain list-of-tokens
    model; after every operation each sequence read through its table must equal
    the model, and the reference counts must be consistent."""
    rng = np.random.default_rng(seed)
    nblk, bs = 12, 4
    pool = RefPool(nblk, bs, rng.permutation(nblk))
    pages = np.full((nblk, bs, 1, 1), -1, dtype=np.int64)  # token ids stand in for K/V bytes
    model = {}
    next_tok = 0
    next_seq = 0
    n_cow = 0
    for _ in range(n_ops):
        live = pool.sequences()
        r = rng.random()
        if r < 0.15 or not live:
            n = int(rng.integers(0, 7))
            try:
                table = pool.alloc(next_seq, n)
            except MemoryError:
                continue
            toks = list(range(next_tok, next_tok + n))
            next_tok += n
            for t, tok in enumerate(toks):
                pages[table[t // bs], t % bs, 0, 0] = tok
            model[next_seq] = toks
            next_seq += 1
        elif r < 0.35:
            parent = live[int(rng.integers(0, len(live)))]
            pool.fork(parent, next_seq)
            model[next_seq] = list(model[parent])
            next_seq += 1
        elif r < 0.5:
            victim = live[int(rng.integers(0, len(live)))]
            pool.free(victim)
            del model[victim]
        else:
            k = int(rng.integers(1, len(live) + 1))
            batch = [live[i] for i in rng.permutation(len(live))[:k]]
            snap = (pool.free_list(), {s: pool.table(s) for s in live}, [pool.refcount(b) for b in range(nblk)])
            try:
                slots, cows = pool.plan_append(batch)
            except MemoryError:
                assert snap == (pool.free_list(), {s: pool.table(s) for s in live},
                                [pool.refcount(b) for b in range(nblk)])
                continue
            n_cow += len(cows)
            new = np.arange(next_tok, next_tok + len(batch), dtype=np.int64).reshape(-1, 1, 1)
            next_tok += len(batch)
            pages, _ = apply_append(pages, pages, slots, cows, new, new)
            for s, tok in zip(batch, new[:, 0, 0]):
                model[s].append(int(tok))
        # every sequence reads back its own history through its table
        refs = [0] * nblk
        for s in pool.sequences():
            t = pool.table(s)
            n = pool.length(s)
            assert n == len(model[s])
            assert len(t) == -(-n // bs)  # only the last block is partly filled
            got = [int(pages[t[i // bs], i % bs, 0, 0]) for i in range(n)]
            assert got == model[s]
            for b in t:
                refs[b] += 1
        free = pool.free_list()
        assert sorted(free + [b for b in range(nblk) if refs[b] > 0]) == list(range(nblk))
        for b in range(nblk):
            assert pool.refcount(b) == refs[b]
            assert (refs[b] == 0) == (b in free)
    assert n_cow > 0  # the walk did exercise copy-on-write


def check_slot_arithmetic(RefPool):
    """Slot of token t = table[t // block_size] * block_size + t % block_size."""
    rng = np.random.default_rng(3)
    for bs in (1, 4, 16):
        pool = RefPool(40, bs, rng.permutation(40))
        pool.alloc("s", 5)
        for _ in range(3 * bs + 2):
            pos = pool.length("s")
            slots, _ = pool.plan_append(["s"])
            t = pool.table("s")
            assert slots[0] == t[pos // bs] * bs + pos % bs
        n = pool.length("s")
        assert len(t) * bs - n <= bs - 1


def check_identical_histories_identical_bytes(RefPool, apply_append, seed=9):
    """Two branches forked at an unaligned length and fed the same tokens read
    back the same bytes, whether their tail block was copied or written in place."""
    rng = np.random.default_rng(seed)
    nblk, bs = 16, 4
    pool = RefPool(nblk, bs, rng.permutation(nblk))
    pages = rng.integers(0, 1 << 16, size=(nblk, bs, 2, 3)).astype(np.uint16)
    pool.alloc("p", 6)
    pool.fork("p", "a")
    pool.fork("p", "b")
    for step in range(7):
        new = rng.integers(0, 1 << 16, size=(1, 2, 3)).astype(np.uint16)
        batch = ["a", "b"] if step % 2 == 0 else ["b", "a"]
        slots, cows = pool.plan_append(batch)
        pages, _ = apply_append(pages, pages, slots, cows, np.repeat(new, 2, 0), np.repeat(new, 2, 0))
    ta, tb = pool.table("a"), pool.table("b")
    n = pool.length("a")
    ra = np.stack([pages[ta[i // bs], i % bs] for i in range(n)])
    rb = np.stack([pages[tb[i // bs], i % bs] for i in range(n)])
    assert np.array_equal(ra, rb)
    assert ta[0] == tb[0] and ta[1] != tb[1]  # full block still shared, tail copied


def run_pool_pins(RefPool, apply_append):
    check_worked_example(RefPool)
    check_error_conventions(RefPool)
    check_slot_arithmetic(RefPool)
    check_pool_against_unpaged_model(RefPool, apply_append)
    check_identical_histories_identical_bytes(RefPool, apply_append)


# ---------------------------------------------------------------------------
# multi-token (extend) attention


def _extend_case(rng, dtype, lens, q_lens, Hq=4, Hkv=2, d=4, block_size=4):
    q_rows = int(sum(q_lens))
    _, k, v, bt, sl = random_paged_case(rng, len(lens), Hq, Hkv, d, block_size, lens, dtype)
    q = to_bits(rng.standard_normal((q_rows, Hq, d)), dtype)
    return q, k, v, bt, sl, np.asarray(q_lens, dtype=np.int32)


def run_extend_pins(ref_extend, ref_decode, bruteforce_decode):
    """Pins for the extend oracle: every query token equals an independent token-by-token
    decode of its row truncated at its own position; one query token per row is plain
    decode; tokens after a query's position never change its output."""
    rng = np.random.default_rng(1234)
    for dtype in ("bf16", "f16"):
        lens, q_lens = [9, 13, 6, 5], [3, 5, 6, 0]  # a row whose every token is a query; a row with none
        q, k, v, bt, sl, ql = _extend_case(rng, dtype, lens, q_lens)
        scale = 0.61
        got = ref_extend(q, k, v, bt, sl, ql, scale, dtype)
        assert got.shape == (sum(q_lens), 4, 4)
        r = 0
        for b, (n, m) in enumerate(zip(lens, q_lens)):
            for i in range(m):
                pos = n - m + i
                one = bruteforce_decode(q[r:r + 1], k, v, bt[b:b + 1], np.asarray([pos + 1]), scale, dtype)
                assert np.max(np.abs(np.asarray(one[0]) - got[r])) < 1e-12, (dtype, b, i)
                r += 1
        # one query token per row: the decode definition
        q1 = to_bits(rng.standard_normal((len(lens), 4, 4)), dtype)
        ones = np.ones(len(lens), dtype=np.int32)
        assert np.max(np.abs(ref_extend(q1, k, v, bt, sl, ones, scale, dtype) -
                             ref_decode(q1, k, v, bt, sl, scale, dtype))) < 1e-13
    # causality: rewrite the tokens after row 1's first query position
    q, k, v, bt, sl, ql = _extend_case(rng, "bf16", [11, 14], [2, 6])
    base = ref_extend(q, k, v, bt, sl, ql, 0.5, "bf16")
    first = 2  # packed index of row 1's first query token
    pos = 14 - 6
    k2, v2 = k.copy(), v.copy()
    for t in range(pos + 1, 14):
        blk, row = int(bt[1, t // 4]), t % 4
        k2[blk, row] = to_bits(rng.standard_normal(k.shape[2:]) * 3, "bf16")
        v2[blk, row] = to_bits(rng.standard_normal(v.shape[2:]) * 3, "bf16")
    moved = ref_extend(q, k2, v2, bt, sl, ql, 0.5, "bf16")
    assert np.array_equal(moved[: first + 1], base[: first + 1])
    assert np.max(np.abs(moved[first + 1:] - base[first + 1:])) > 1e-3

"""Pins for the pool's swap space (reading R7 of oracle/pool.py): a random walk
on tiny pools against an un-paged list-of-tokens model, with every sequence,
resident or swapped out, read back through its placement after every step;
reference and slot accounting; closed-form counts; and decode before a swap-out
equal to decode after the swap-in, bit for bit."""

import numpy as np

import oracle_checks as oc


def _read(pool, seq, pages, host_pages, bs):
    n = pool.length(seq)
    place = pool.placement(seq)
    assert len(place) == -(-n // bs)
    out = []
    for i in range(n):
        kind, x = place[i // bs]
        src = host_pages if kind == "host" else pages
        out.append(int(src[x, i % bs, 0, 0]))
    return out


def check_swap_against_unpaged_model(RefPool, apply_append, apply_swap, seed=0, n_ops=500):
    rng = np.random.default_rng(seed)
    nblk, nhost, bs = 14, 10, 4
    pool = RefPool(nblk, bs, rng.permutation(nblk), nhost, rng.permutation(nhost))
    pages = np.full((nblk, bs, 1, 1), -1, dtype=np.int64)
    host = np.full((nhost, bs, 1, 1), -2, dtype=np.int64)
    model, nxt_tok, nxt_seq = {}, 0, 0
    counts = {"out": 0, "in": 0, "shared_kept": 0}
    for _ in range(n_ops):
        seqs = sorted(model)
        resident = [s for s in seqs if not pool.is_swapped(s)]
        swapped = [s for s in seqs if pool.is_swapped(s)]
        r = rng.random()
        if r < 0.15 or not seqs:
            n = int(rng.integers(0, 9))
            try:
                pool.alloc(nxt_seq, n)
            except MemoryError:
                continue
            table = pool.table(nxt_seq)
            for t in range(n):
                pages[table[t // bs], t % bs, 0, 0] = nxt_tok + t
            model[nxt_seq] = list(range(nxt_tok, nxt_tok + n))
            nxt_tok += n
            nxt_seq += 1
        elif r < 0.27 and resident:
            parent = resident[int(rng.integers(len(resident)))]
            pool.fork(parent, nxt_seq)
            model[nxt_seq] = list(model[parent])
            nxt_seq += 1
        elif r < 0.37:
            victim = seqs[int(rng.integers(len(seqs)))]
            pool.free(victim)
            del model[victim]
        elif r < 0.55 and resident:
            s = resident[int(rng.integers(len(resident)))]
            before = (pool.free_list(), pool.host_free_list(), [pool.refcount(b) for b in range(nblk)])
            try:
                copies = pool.swap_out(s)
            except MemoryError:
                assert before == (pool.free_list(), pool.host_free_list(), [pool.refcount(b) for b in range(nblk)])
                continue
            host = apply_swap(host, pages, copies)
            pages[[b for b, _ in copies]] = -3          # the freed device blocks may be reused: poison them
            counts["out"] += 1
            counts["shared_kept"] += sum(1 for kind, _ in pool.placement(s) if kind == "device")
        elif r < 0.72 and swapped:
            s = swapped[int(rng.integers(len(swapped)))]
            before = (pool.free_list(), pool.host_free_list(), [pool.refcount(b) for b in range(nblk)])
            try:
                copies = pool.swap_in(s)
            except MemoryError:
                assert before == (pool.free_list(), pool.host_free_list(), [pool.refcount(b) for b in range(nblk)])
                continue
            pages = apply_swap(pages, host, copies)
            host[[h for h, _ in copies]] = -4
            counts["in"] += 1
        elif resident:
            k = int(rng.integers(1, len(resident) + 1))
            batch = [resident[i] for i in rng.permutation(len(resident))[:k]]
            try:
                slots, cows = pool.plan_append(batch)
            except MemoryError:
                continue
            new = np.arange(nxt_tok, nxt_tok + len(batch), dtype=np.int64).reshape(-1, 1, 1)
            nxt_tok += len(batch)
            pages, _ = apply_append(pages, pages, slots, cows, new, new)
            for s, tok in zip(batch, new[:, 0, 0]):
                model[s].append(int(tok))
        # every sequence reads back its history; counts and slots are consistent
        refs, host_used = [0] * nblk, []
        for s in sorted(model):
            assert _read(pool, s, pages, host, bs) == model[s]
            for kind, x in pool.placement(s):
                if kind == "host":
                    host_used.append(x)
                else:
                    refs[x] += 1
        assert [pool.refcount(b) for b in range(nblk)] == refs
        assert sorted(pool.free_list()) == [b for b in range(nblk) if refs[b] == 0]
        assert len(set(host_used)) == len(host_used)
        assert sorted(pool.host_free_list() + host_used) == list(range(nhost))
    assert counts["out"] > 5 and counts["in"] > 5 and counts["shared_kept"] > 0, counts


def check_swap_closed_forms(RefPool):
    """A sequence holding 5 blocks alone and sharing 3 (a fork's prefix):
    swap-out moves exactly the 5, frees them to the back of the device list in
    table order and takes host slots from the front; swap-in takes 5 device
    blocks from the front and returns the slots; both fail whole on shortage."""
    bs = 4
    pool = RefPool(20, bs, list(range(20)), 8, list(range(8)))
    pool.alloc(100, 3 * bs)                      # blocks 0, 1, 2
    pool.fork(100, 101)
    pool.plan_append([101])                         # block 3
    for _ in range(5 * bs - 1):
        pool.plan_append([101])                     # blocks 4..7
    assert pool.table(101) == [0, 1, 2, 3, 4, 5, 6, 7]
    copies = pool.swap_out(101)
    assert copies == [(3, 0), (4, 1), (5, 2), (6, 3), (7, 4)]
    assert pool.placement(101) == [("device", 0), ("device", 1), ("device", 2)] + [("host", h) for h in range(5)]
    assert pool.free_list() == list(range(8, 20)) + [3, 4, 5, 6, 7]
    assert pool.host_free_list() == [5, 6, 7]
    assert [pool.refcount(b) for b in range(3)] == [2, 2, 2]
    for bad in (lambda: pool.plan_append([101]), lambda: pool.fork(101, 102), lambda: pool.table(101),
                lambda: pool.export_tables([101], 8), lambda: pool.swap_out(101)):
        try:
            bad()
        except (ValueError, KeyError):
            pass
        else:
            raise AssertionError("an operation on a swapped-out sequence was accepted")
    try:
        pool.swap_in(100)
    except (ValueError, KeyError):
        pass
    else:
        raise AssertionError("swap_in of a resident sequence was accepted")
    pool.alloc(103, 14 * bs)                   # leaves 3 device blocks: too few to swap 101 in
    snap = (pool.free_list(), pool.host_free_list())
    oc.expect_error(MemoryError, pool.swap_in, 101)
    assert snap == (pool.free_list(), pool.host_free_list())
    pool.free(103)
    assert pool.free_list() == [5, 6, 7] + list(range(8, 20)) + [3, 4]
    copies = pool.swap_in(101)
    assert copies == [(0, 5), (1, 6), (2, 7), (3, 8), (4, 9)]
    assert pool.table(101) == [0, 1, 2, 5, 6, 7, 8, 9]
    assert pool.host_free_list() == [5, 6, 7, 0, 1, 2, 3, 4]
    # host shortage: a 9-block private sequence needs 9 of 8 slots
    pool.alloc(104, 9 * bs)
    snap = (pool.free_list(), pool.host_free_list())
    oc.expect_error(MemoryError, pool.swap_out, 104)
    assert snap == (pool.free_list(), pool.host_free_list())
    # freeing a swapped-out sequence returns its slots and drops its shared references
    pool.swap_out(101)
    pool.free(101)
    assert pool.host_free_count() == 8 and [pool.refcount(b) for b in range(3)] == [1, 1, 1]


def check_swap_preserves_attention(RefPool, apply_append, apply_swap, ref_decode, seed=3):
    """Attention depends only on a sequence's logical tokens: decode before a
    swap-out equals decode after the swap-in bit for bit, though the blocks
    came back at other physical places."""
    rng = np.random.default_rng(seed)
    bs, Hkv, d, Hq = 4, 2, 8, 4
    pool = RefPool(24, bs, rng.permutation(24), 12)
    k = rng.integers(0, 1 << 16, size=(24, bs, Hkv, d), dtype=np.uint64).astype(np.uint16) & 0x3FFF
    v = rng.integers(0, 1 << 16, size=(24, bs, Hkv, d), dtype=np.uint64).astype(np.uint16) & 0x3FFF
    hk = np.zeros((12, bs, Hkv, d), dtype=np.uint16)
    hv = np.zeros_like(hk)
    pool.alloc(0, 13)
    pool.fork(0, 1)
    pool.plan_append([1])
    for _ in range(6):
        slots, cows = pool.plan_append([1])
        new = rng.integers(0, 0x3FFF, size=(1, Hkv, d)).astype(np.uint16)
        k, v = apply_append(k, v, slots, cows, new, new)
    q = rng.integers(0, 0x3FFF, size=(1, Hq, d)).astype(np.uint16)
    bt, lens = pool.export_tables([1], 8)
    before = ref_decode(q, k, v, bt, lens, 0.3, "bf16")
    old = pool.table(1)
    copies = pool.swap_out(1)
    hk, hv = apply_swap(hk, k, copies), apply_swap(hv, v, copies)
    k[[b for b, _ in copies]] = 0x7F80                # reused blocks: overwrite (bf16 +Inf)
    v[[b for b, _ in copies]] = 0x7F80
    pool.alloc(2, len(copies) * bs)                   # someone takes the freed blocks
    back = pool.swap_in(1)
    k, v = apply_swap(k, hk, back), apply_swap(v, hv, back)
    assert pool.table(1) != old
    bt, lens = pool.export_tables([1], 8)
    after = ref_decode(q, k, v, bt, lens, 0.3, "bf16")
    assert np.array_equal(before, after)


def run_swap_pins(RefPool, apply_append, apply_swap, ref_decode):
    check_swap_closed_forms(RefPool)
    check_swap_against_unpaged_model(RefPool, apply_append, apply_swap)
    check_swap_preserves_attention(RefPool, apply_append, apply_swap, ref_decode)

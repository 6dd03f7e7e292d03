"""The library's swap space (pkv_seq_swap_out / pkv_seq_swap_in and the pool calls
around them) against the oracle pool: the same random walks give identical copy
lists, placements, counts and free lists; the closed forms and the un-paged token
model hold for the library as well.  No GPU: copies are applied on the host."""

import numpy as np
import pytest

import swap_checks as sc
from oracle import RefPool, apply_append
from oracle.pool import apply_swap

pk = pytest.importorskip("paged_kv_cache_21_amd")


def test_closed_forms_on_the_library():
    sc.check_swap_closed_forms(pk.BlockPool)


@pytest.mark.parametrize("seed", range(3))
def test_library_against_unpaged_model(seed):
    sc.check_swap_against_unpaged_model(pk.BlockPool, apply_append, apply_swap, seed=seed)


@pytest.mark.parametrize("seed", range(6))
def test_random_walk_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    nblk, nhost, bs = 24, 16, 4
    order, horder = rng.permutation(nblk), rng.permutation(nhost)
    lib = pk.BlockPool(nblk, bs, order, nhost, horder)
    ora = RefPool(nblk, bs, order, nhost, horder)
    seqs, nxt = [], 0

    def both(name, *args):
        out = []
        for p in (lib, ora):
            try:
                r = getattr(p, name)(*args)
                out.append(("ok", r if name.startswith("swap") else None))
            except MemoryError:
                out.append(("oom", None))
            except ValueError:
                out.append(("invalid", None))
            except KeyError:
                out.append(("not found", None))
        assert out[0] == out[1], (name, args, out)
        return out[0]

    for step in range(400):
        r = rng.random()
        if r < 0.2 or not seqs:
            if both("alloc", nxt, int(rng.integers(0, 14)))[0] == "ok":
                seqs.append(nxt)
            nxt += 1
        elif r < 0.3:
            if both("fork", seqs[rng.integers(len(seqs))], nxt)[0] == "ok":
                seqs.append(nxt)
            nxt += 1
        elif r < 0.4:
            s = seqs.pop(int(rng.integers(len(seqs))))
            both("free", s)
        elif r < 0.55:
            both("swap_out", seqs[rng.integers(len(seqs))])
        elif r < 0.7:
            both("swap_in", seqs[rng.integers(len(seqs))])
        else:
            k = int(rng.integers(1, len(seqs) + 1))
            batch = [seqs[i] for i in rng.permutation(len(seqs))[:k]]
            res = []
            for p in (lib, ora):
                try:
                    sl, cows = p.plan_append(batch)
                    res.append((list(sl), [tuple(int(x) for x in c) for c in cows]))
                except MemoryError:
                    res.append("oom")
                except ValueError:
                    res.append("err")
            assert res[0] == res[1]
        for s in seqs:
            assert lib.placement(s) == ora.placement(s)
            assert lib.is_swapped(s) == ora.is_swapped(s)
        assert lib.free_list() == ora.free_list()
        assert lib.host_free_list() == ora.host_free_list()
        assert [lib.refcount(b) for b in range(nblk)] == [ora.refcount(b) for b in range(nblk)]


def test_swapped_sequence_cannot_be_cached():
    pool = pk.BlockPool(16, 4, None, 8)
    cache = pk.RadixCache(pool)
    got = cache.admit([[1, 2, 3, 4, 5, 6, 7, 8, 9]], [7])
    pool.swap_out(7)
    with pytest.raises(ValueError):
        cache.finish([[1, 2, 3, 4, 5, 6, 7, 8, 9]], [7], [got[0][1]])
    pool.swap_in(7)
    cache.finish([[1, 2, 3, 4, 5, 6, 7, 8, 9]], [7], [got[0][1]])
    assert cache.cached_blocks() == 2

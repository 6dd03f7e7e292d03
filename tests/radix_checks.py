"""Checks for the prefix cache (radix tree over pool blocks).

``FlatModel`` is an independent model of the cache that knows nothing of tree
nodes: the set of cached block paths (every cached prefix, one entry per block)
with the block id, last access time, lock count, score and depth of each.
Longest match is a brute-force walk over that set, and an eviction is checked
against a brute-force minimum over all unlocked leaf paths.  ``PinnedCache``
runs an oracle cache beside the flat model and asserts after every call that
the two hold the same state and that the pool's reference counts equal the
references that the tree and the live sequences hold.

``TraceDriver`` generates seeded request traces (arrivals that reuse earlier
prefixes, finished requests cached, multi-turn continuation, evictions under
pool pressure, score updates, plain lookups) against any object with the
cache's method names, so the same traces pin the oracle and compare the
library with it.
"""

from collections import defaultdict

import numpy as np


def cut(tokens, bs):
    tokens = [int(t) for t in tokens]
    return [tuple(tokens[i * bs:(i + 1) * bs]) for i in range(len(tokens) // bs)]


def expand(cache, bs):
    """{block path: (block, time, lock, score, depth)} and {node id: its end path}."""
    ids = cache.node_ids()
    info = {i: cache.node_info(i) for i in ids}
    children = defaultdict(list)
    for i in ids:
        if info[i][0] >= 0:
            children[info[i][0]].append(i)
    paths, end = {}, {0: ()}
    stack = [0]
    while stack:
        i = stack.pop()
        if i != 0:
            parent, blocks, lock, stamp, score, depth = info[i]
            key = cut(cache.node_tokens(i), bs)
            assert len(key) == len(blocks) >= 1, f"node {i}: {len(key)} key blocks, {len(blocks)} ids"
            p = end[parent]
            for blk, b in zip(key, blocks):
                p = p + (blk,)
                assert p not in paths, f"block path cached twice (node {i})"
                paths[p] = (b, stamp, lock, score, depth)
            end[i] = p
        stack.extend(children[i])
    assert set(end) == set(ids), "nodes unreachable from the root"
    return paths, end


class FlatModel:
    def __init__(self, bs, policy):
        self.bs = bs
        self.policy = policy
        self.paths = {}   # path -> [block, time, lock, score, depth]
        self.clock = 0

    def longest(self, key):
        k = 0
        while k < len(key) and tuple(key[:k + 1]) in self.paths:
            k += 1
        return k

    def match(self, tokens):
        self.clock += 1
        key = cut(tokens, self.bs)
        k = self.longest(key)
        for j in range(1, k + 1):
            self.paths[tuple(key[:j])][1] = self.clock
        return k * self.bs, [self.paths[tuple(key[:j])][0] for j in range(1, k + 1)]

    def insert(self, tokens, blocks, score, depth):
        self.clock += 1
        key = cut(tokens, self.bs)
        adopted = []
        for j in range(1, len(key) + 1):
            p = tuple(key[:j])
            if p in self.paths:
                self.paths[p][1] = self.clock
                self.paths[p][3] = max(self.paths[p][3], float(score))
            else:
                self.paths[p] = [int(blocks[j - 1]), self.clock, 0, float(score), int(depth)]
                adopted.append(int(blocks[j - 1]))
        return adopted

    def lock(self, end_path, delta):
        for j in range(1, len(end_path) + 1):
            self.paths[end_path[:j]][2] += delta
            assert self.paths[end_path[:j]][2] >= 0

    def set_score(self, own_paths, ancestor_end, score):
        for p in own_paths:
            self.paths[p][3] = float(score)
        for j in range(1, len(ancestor_end) + 1):
            self.paths[ancestor_end[:j]][3] = max(self.paths[ancestor_end[:j]][3], float(score))

    def order_key(self, p):
        block, stamp, lock, score, depth = self.paths[p]
        if self.policy == "lru":
            return (stamp,)
        return (score / (depth + 1), stamp)

    def check_and_remove_victim(self, victim_paths):
        """The victim (a node's block paths) must end in an unlocked leaf path whose
        order key is the minimum over all unlocked leaf paths; removes it."""
        parents = {p[:-1] for p in self.paths}
        leaves = [p for p in self.paths if p not in parents and self.paths[p][2] == 0]
        deepest = max(victim_paths, key=len)
        assert deepest in leaves, "evicted a node that is not an unlocked leaf"
        assert all(self.paths[p][2] == 0 for p in victim_paths), "evicted a locked block"
        best = min(self.order_key(p) for p in leaves)
        assert self.order_key(deepest) == best, f"eviction order: took {self.order_key(deepest)}, best {best}"
        blocks = [self.paths[p][0] for p in sorted(victim_paths, key=len)]
        for p in victim_paths:
            del self.paths[p]
        return blocks

    def state(self):
        return {p: tuple(v) for p, v in self.paths.items()}


def check_pool_accounting(pool, cache, bs, live_seqs):
    """Counts = tree references + sequence references; free list = blocks at 0."""
    paths, _ = expand(cache, bs)
    tree_blocks = [v[0] for v in paths.values()]
    assert len(set(tree_blocks)) == len(tree_blocks), "a block is cached at two paths"
    expect = [0] * pool.num_blocks
    for b in tree_blocks:
        expect[b] += 1
    for s in live_seqs:
        for b in pool.table(s):
            expect[b] += 1
    got = [pool.refcount(b) for b in range(pool.num_blocks)]
    assert got == expect, "reference counts differ from the references held"
    free = pool.free_list()
    assert sorted(free) == [b for b in range(pool.num_blocks) if expect[b] == 0], "free list is not the unused blocks"
    assert cache.cached_blocks() == len(tree_blocks)
    assert cache.evictable_blocks() == sum(1 for v in paths.values() if v[2] == 0)


class PinnedCache:
    """An oracle cache driven in lockstep with FlatModel (same method names)."""

    def __init__(self, pool, cache, bs, policy):
        self.pool, self.cache, self.bs = pool, cache, bs
        self.flat = FlatModel(bs, policy)
        self.live = set()

    def _check(self):
        paths, _ = expand(self.cache, self.bs)
        assert {p: v for p, v in paths.items()} == self.flat.state(), "cache state differs from the flat model"
        check_pool_accounting(self.pool, self.cache, self.bs, self.live)

    # cache calls
    def match_prefix(self, tokens):
        m, blocks, node = self.cache.match_prefix(tokens)
        fm, fblocks = self.flat.match(tokens)
        assert (m, blocks) == (fm, fblocks), f"match {m} {blocks} != brute force {fm} {fblocks}"
        _, end = expand(self.cache, self.bs)
        assert len(end[node]) * self.bs == m, "match node does not end at the match"
        self._check()
        return m, blocks, node

    def insert(self, tokens, blocks, score=0.0, depth=0):
        before = self.pool.free_count()
        node, adopted = self.cache.insert(tokens, blocks, score, depth)
        fadopted = self.flat.insert(tokens, blocks, score, depth)
        assert adopted == len(fadopted)
        assert self.pool.free_count() == before
        _, end = expand(self.cache, self.bs)
        assert len(end[node]) == len(cut(tokens, self.bs)), "insert node does not end at the last full block"
        self._check()
        return node, adopted

    def lock(self, node):
        _, end = expand(self.cache, self.bs)
        self.cache.lock(node)
        self.flat.lock(end[node], +1)
        self._check()

    def unlock(self, node):
        _, end = expand(self.cache, self.bs)
        self.cache.unlock(node)
        self.flat.lock(end[node], -1)
        self._check()

    def set_score(self, node, score):
        _, end = expand(self.cache, self.bs)
        parent = self.cache.node_info(node)[0]
        own = [end[node][:j] for j in range(len(end[parent]) + 1, len(end[node]) + 1)]
        self.cache.set_score(node, score)
        self.flat.set_score(own, end[parent], score)
        self._check()

    def evict(self, num_blocks):
        paths_before, end_before = expand(self.cache, self.bs)
        parent_of = {i: self.cache.node_info(i)[0] for i in self.cache.node_ids()}
        free_before = self.pool.free_list()
        released, evicted = self.cache.evict(num_blocks)
        freed = []
        for v in evicted:
            p0 = end_before[parent_of[v]]
            own = [end_before[v][:j] for j in range(len(p0) + 1, len(end_before[v]) + 1)]
            for b in self.flat.check_and_remove_victim(own):
                # a block goes back to the free list when no sequence still holds it
                if not any(b in self.pool.table(s) for s in self.live):
                    freed.append(b)
        assert self.pool.free_list() == free_before + freed, "released blocks or their order differ"
        assert released == len(freed)
        if released < num_blocks:
            parents = {p[:-1] for p in self.flat.paths}
            assert not any(p not in parents and self.flat.paths[p][2] == 0 for p in self.flat.paths), \
                "stopped with unlocked leaves left"
        self._check()
        return released, evicted

    def node_ids(self):
        return self.cache.node_ids()

    def node_info(self, node):
        return self.cache.node_info(node)

    # batched calls, taken step by step through the checked calls above
    def admit(self, requests, seqs):
        out = []
        for toks, seq in zip(requests, seqs):
            m, blocks, node = self.match_prefix(list(toks)[:-1])
            self.lock(node)
            need = -(-len(toks) // self.bs) - len(blocks)
            if need > self.pool.free_count():
                self.evict(need - self.pool.free_count())
            try:
                self.alloc_with_prefix(seq, blocks, len(toks))
            except MemoryError:
                self.unlock(node)
                break
            out.append((m, node))
        return out

    def finish(self, requests, seqs, nodes, scores, depths):
        for toks, seq, node, sc, dp in zip(requests, seqs, nodes, scores, depths):
            self.insert(toks, self.pool.table(seq), sc, dp)
            self.unlock(node)
            self.free(seq)

    # pool calls the request traces make
    def alloc_with_prefix(self, seq, blocks, n):
        self.pool.alloc_with_prefix(seq, blocks, n)
        self.live.add(seq)
        self._check()

    def free(self, seq):
        self.pool.free(seq)
        self.live.discard(seq)
        self._check()

    def plan_append(self, seqs):
        out = self.pool.plan_append(seqs)
        self._check()
        return out

    def table(self, seq):
        return self.pool.table(seq)


class TraceDriver:
    """Seeded request trace against ``sys`` (cache + pool calls by name)."""

    def __init__(self, sys, bs, seed, vocab=3, max_blocks=6):
        self.sys, self.bs = sys, bs
        self.rng = np.random.default_rng(seed)
        self.vocab, self.max_blocks = vocab, max_blocks
        self.active = {}    # seq -> [tokens, locked node]
        self.history = []
        self.next_seq = 0
        self.log = []
        self.batched = hasattr(sys, "admit")

    def _tokens(self):
        rng = self.rng
        base = []
        if self.history and rng.random() < 0.75:
            src = self.history[rng.integers(len(self.history))]
            base = src[:rng.integers(0, len(src) + 1)]
        total = max(len(base) + int(rng.integers(1, 2 * self.bs + 1)), 1)
        total = min(total, self.max_blocks * self.bs)
        extra = [int(x) for x in rng.integers(0, self.vocab, size=max(total - len(base), 0))]
        return list(base[:total]) + extra

    def arrive(self):
        toks = self._tokens()
        m, blocks, node = self.sys.match_prefix(toks[:-1])
        if self.rng.random() < 0.2:
            node = None     # a reader that holds its blocks without locking the tree
        else:
            self.sys.lock(node)
        seq = self.next_seq
        self.next_seq += 1
        try:
            self.sys.alloc_with_prefix(seq, blocks, len(toks))
        except MemoryError:
            if node is None:         # an unlocked reader could evict its own prefix: give up
                self.log.append(("drop", seq))
                return
            need = -(-len(toks) // self.bs) - len(blocks)
            self.sys.evict(need)
            try:
                self.sys.alloc_with_prefix(seq, blocks, len(toks))
            except MemoryError:
                if node is not None:
                    self.sys.unlock(node)
                self.log.append(("drop", seq))
                return
        self.active[seq] = [toks, node]
        self.history.append(toks)
        self.log.append(("arrive", seq, m))

    def finish(self):
        seq = sorted(self.active)[self.rng.integers(len(self.active))]
        toks, node = self.active.pop(seq)
        score = float(self.rng.integers(0, 8)) / 4.0
        depth = int(self.rng.integers(0, 4))
        new_node, adopted = self.sys.insert(toks, self.sys.table(seq), score, depth)
        if node is not None:
            self.sys.unlock(node)
        self.sys.free(seq)
        self.log.append(("finish", seq, new_node, adopted))

    def turn(self):
        seq = sorted(self.active)[self.rng.integers(len(self.active))]
        toks, node = self.active[seq]
        new_node, _ = self.sys.insert(toks, self.sys.table(seq), 0.0, 0)
        self.sys.lock(new_node)
        if node is not None:
            self.sys.unlock(node)
        self.active[seq][1] = new_node
        grow = int(self.rng.integers(1, self.bs + 2))
        for _ in range(grow):
            if len(toks) >= self.max_blocks * self.bs:
                break
            try:
                self.sys.plan_append([seq])
            except MemoryError:
                self.sys.evict(1)
                try:
                    self.sys.plan_append([seq])
                except MemoryError:
                    break
            toks.append(int(self.rng.integers(0, self.vocab)))
        self.history.append(list(toks))
        self.log.append(("turn", seq, new_node))

    def batch(self):
        """Admit a few requests in one call, then finish a few active ones in one call."""
        reqs = [self._tokens() for _ in range(int(self.rng.integers(1, 5)))]
        seqs = list(range(self.next_seq, self.next_seq + len(reqs)))
        self.next_seq += len(reqs)
        got = self.sys.admit(reqs, seqs)
        for (m, node), toks, seq in zip(got, reqs, seqs):
            self.active[seq] = [toks, node]
            self.history.append(toks)
        self.log.append(("admit", len(reqs), len(got)) + tuple(m for m, _ in got))
        done = [s for s in sorted(self.active) if self.active[s][1] is not None]
        if done:
            k = int(self.rng.integers(1, min(4, len(done)) + 1))
            pick = [done[i] for i in sorted(self.rng.choice(len(done), size=k, replace=False))]
            toks = [self.active[s][0] for s in pick]
            nodes = [self.active[s][1] for s in pick]
            scores = [float(self.rng.integers(0, 8)) / 4.0 for _ in pick]
            depths = [int(self.rng.integers(0, 4)) for _ in pick]
            self.sys.finish(toks, pick, nodes, scores, depths)
            for s in pick:
                del self.active[s]
            self.log.append(("finish_batch",) + tuple(pick))

    def step(self):
        r = self.rng.random()
        if self.batched and r < 0.15:
            self.batch()
        elif r < 0.35 or not self.active:
            self.arrive()
        elif r < 0.6:
            self.finish()
        elif r < 0.72:
            self.turn()
        elif r < 0.82:
            n = int(self.rng.integers(0, 6))
            self.log.append(("evict", n) + tuple(self.sys.evict(n)))
        elif r < 0.92:
            ids = [i for i in self.sys.node_ids() if i != 0]
            if ids:
                node = ids[self.rng.integers(len(ids))]
                s = float(self.rng.integers(0, 8)) / 4.0
                self.sys.set_score(node, s)
                self.log.append(("score", node, s))
        else:
            if self.history:
                src = self.history[self.rng.integers(len(self.history))]
                self.log.append(("query",) + tuple(self.sys.match_prefix(src)[:1]))

    def run(self, steps):
        for _ in range(steps):
            self.step()
        return self.log


# ---------------------------------------------------------------------------
# scenarios from the pages, with their closed-form outcomes


def scenario_system_prompt(Cache, Pool, users=1000, prompt=2000, bs=16, seed=0):
    """One long system prompt shared by every user's request ("RadixAttention":
    1,000 users whose requests start with the same 2,000-token prompt): after the
    first request is cached, each later one matches the whole prompt (2,000 =
    125 blocks of 16), points at the same blocks and caches only its own full
    blocks."""
    rng = np.random.default_rng(seed)
    user_len = rng.integers(1, 65, size=users)
    pool = Pool(125 + int(sum(user_len // bs)) + 8, bs)
    cache = Cache(pool, "lru")
    sys_prompt = [int(x) for x in rng.integers(0, 50_000, size=prompt)]
    hits = 0
    first_blocks = None
    for u in range(users):
        toks = sys_prompt + [50_000 + u * 100 + i for i in range(int(user_len[u]))]
        m, blocks, node = cache.match_prefix(toks[:-1])
        if u == 0:
            assert (m, blocks, node) == (0, [], 0)
        else:
            assert m == prompt and blocks == first_blocks, (u, m)
        hits += m
        cache.lock(node)
        pool.alloc_with_prefix(u, blocks, len(toks))
        table = pool.table(u)
        _, adopted = cache.insert(toks, table)
        assert adopted == len(toks) // bs - m // bs
        if u == 0:
            first_blocks = table[:prompt // bs]
        cache.unlock(node)
        pool.free(u)
        # the tree keeps exactly one reference to every cached block once the request is gone
        assert all(pool.refcount(b) == 1 for b in first_blocks), ("cached prompt blocks lost their reference", u)
    assert hits == (users - 1) * prompt
    assert cache.cached_blocks() == prompt // bs + int(sum(user_len // bs))
    for b in first_blocks:
        assert pool.refcount(b) == 1
    return hits


def scenario_multi_turn(Cache, Pool, bs=4, turns=5, seed=1):
    """Each turn of a conversation resends the whole history ("RadixAttention":
    turn 5 only appends to the leaf that turn 4 left): turn k+1 matches turn k's
    cached blocks exactly, and its insert hangs one new leaf under turn k's node."""
    rng = np.random.default_rng(seed)
    pool = Pool(256, bs)
    cache = Cache(pool, "lru")
    history, prev_node = [], 0
    for t in range(turns):
        history = history + [int(x) for x in rng.integers(0, 1000, size=int(rng.integers(bs, 4 * bs)))]
        m, blocks, node = cache.match_prefix(history)
        if t > 0:
            assert node == prev_node
            assert m == (len(prev_hist) // bs) * bs
        pool.alloc_with_prefix(t, blocks, len(history))
        new_node, adopted = cache.insert(history, pool.table(t))
        assert adopted == len(history) // bs - m // bs
        if adopted:
            assert cache.node_info(new_node)[0] == prev_node
            prev_node = new_node
        pool.free(t)
        prev_hist = list(history)
    # one node per turn that added a full block, chained
    return prev_node


def scenario_branch_and_backtrack(Cache, Pool, bs=4):
    """An agent forks its state, explores branch A, goes back to the fork and
    explores branch B ("RadixAttention": no recomputation of the shared
    context): B matches the whole shared context, A and B are sibling leaves
    under the context's node, and evicting one branch keeps the context."""
    pool = Pool(64, bs)
    cache = Cache(pool, "lru")
    ctx = list(range(100, 100 + 5 * bs))
    a = ctx + [1] * (2 * bs)
    b = ctx + [2] * (3 * bs)
    pool.alloc(0, len(a))
    node_a, _ = cache.insert(a, pool.table(0))
    pool.free(0)
    m, blocks, node = cache.match_prefix(b)
    assert m == len(ctx)
    cache.lock(node)
    pool.alloc_with_prefix(1, blocks, len(b))
    node_b, adopted = cache.insert(b, pool.table(1))
    assert adopted == 3
    cache.unlock(node)
    pool.free(1)
    ctx_node = cache.node_info(node_b)[0]
    assert cache.node_info(node_a)[0] == ctx_node == node
    assert cache.node_tokens(ctx_node) == ctx
    cache.lock(node_b)
    released, evicted = cache.evict(1)
    assert evicted == [node_a] and released == 2
    assert cache.match_prefix(b)[0] == len(b)


def scenario_leaf_only_eviction(Cache, Pool, bs=4):
    """Eviction strikes only unlocked leaves, least recently used first, so a
    shared prefix stays while a request uses it ("RadixAttention")."""
    pool = Pool(40, bs)
    cache = Cache(pool, "lru")
    prompt = list(range(1000, 1000 + 3 * bs))
    users = [prompt + [u] * (2 * bs) for u in range(3)]
    nodes = []
    for u, toks in enumerate(users):
        m, blocks, _ = cache.match_prefix(toks)
        pool.alloc_with_prefix(u, blocks, len(toks))
        nodes.append(cache.insert(toks, pool.table(u))[0])
        pool.free(u)
    assert cache.cached_blocks() == 3 + 3 * 2
    cache.match_prefix(users[0])          # user 0 becomes the most recent
    cache.lock(nodes[1])                  # user 1 is in flight
    # a lock covers the node and every ancestor below the root ("lock_ref" on the path)
    n = nodes[1]
    while n != 0:
        parent, _, lock_ref, _, _, _ = cache.node_info(n)
        assert lock_ref == 1, ("lock does not reach node", n)
        n = parent
    released, evicted = cache.evict(100)
    assert evicted == [nodes[2], nodes[0]] and released == 4
    assert cache.cached_blocks() == 3 + 2
    assert cache.match_prefix(users[1])[0] == len(users[1])
    cache.unlock(nodes[1])
    released, evicted = cache.evict(100)
    assert evicted[0] == nodes[1] and released == 5 and cache.cached_blocks() == 0
    assert pool.free_count() == 40


def scenario_evict_blocks_in_use(Cache, Pool, bs=4):
    """Evicting a leaf drops only the tree's references: blocks that a sequence
    still holds stay allocated and reach the free list when that sequence goes."""
    pool = Pool(16, bs)
    cache = Cache(pool, "lru")
    pool.alloc(0, 3 * bs)
    t0 = pool.table(0)
    node, _ = cache.insert(list(range(3 * bs)), t0)
    assert [pool.refcount(b) for b in t0] == [2, 2, 2]
    released, evicted = cache.evict(1)
    assert evicted == [node] and released == 0 and cache.cached_blocks() == 0
    assert [pool.refcount(b) for b in t0] == [1, 1, 1] and pool.free_count() == 16 - 3
    pool.free(0)
    assert pool.free_list()[-3:] == t0


def scenario_batched_admission(Cache, Pool, bs=16):
    """Batched admission (reading K9).  100 users behind a 2,000-token prompt in
    batches of 10: nothing is cached until the first batch finishes, so its 10
    requests match nothing; every later request matches the whole prompt.  A pool
    with room for the cached prompt plus a few tails admits requests while free
    blocks and evictable leaves last, and releases the lock of the first request
    that does not fit."""
    import workloads

    reqs = [[int(t) for t in r] for r in workloads.system_prompt_requests(
        seed=5, users=100, prompt_tokens=2000, user_lo=16, user_hi=16)]   # 2,016 tokens: 126 blocks each
    pool = Pool(126 * 10 + 8, bs)
    cache = Cache(pool, "lru")
    for b in range(10):
        ids = list(range(10 * b, 10 * b + 10))
        got = cache.admit([reqs[i] for i in ids], ids)
        assert len(got) == 10
        assert [m for m, _ in got] == ([0] * 10 if b == 0 else [2000] * 10), (b, got)
        cache.finish([reqs[i] for i in ids], ids, [n for _, n in got])
    # the prompt (125 blocks) and one 16-token tail block per user, all unlocked again
    assert cache.cached_blocks() == 125 + 100 == cache.evictable_blocks()
    # a repeated request leaves its last block to compute: 2,000 of its 2,016 tokens match
    again = cache.admit([reqs[0]], [500])
    assert again[0][0] == 2000
    cache.finish([reqs[0]], [500], [again[0][1]])
    pool2 = Pool(125 + 1 + 4, bs)
    cache2 = Cache(pool2, "lru")
    first = cache2.admit([reqs[0]], [1000])
    cache2.finish([reqs[0]], [1000], [first[0][1]])       # prompt + 1 tail cached: 126 blocks, 4 free
    prompt_node = cache2.match_prefix(reqs[1][:2000])[2]
    got = cache2.admit([reqs[i] for i in range(1, 9)], list(range(2001, 2009)))
    # each request needs 1 fresh block: 4 free ones, then the first tail's leaf is evicted -> 5 admitted
    assert len(got) == 5 and all(m == 2000 for m, _ in got), got
    assert cache2.node_info(prompt_node)[2] == 5          # the 6th request's lock was released
    for bad in (([reqs[1]], [2001], [10 ** 9]),            # no such node
                ([reqs[1], reqs[1]], [2001, 2001], [got[0][1]] * 2)):   # repeated sequence
        try:
            cache2.finish(*bad)
        except (ValueError, KeyError):
            pass
        else:
            raise AssertionError(f"finish accepted {bad[1]}")
    assert cache2.node_info(prompt_node)[2] == 5 and pool2.free_count() == 0


def scenario_rsbcm_order(Cache, Pool, bs=2):
    """RSBCM ("RKSC", §2 C): blocks go in order of branch_score / (depth + 1),
    lowest first.  Three leaves with (score, depth) = (0.9, 1), (0.3, 0),
    (0.8, 3) have importance 0.45, 0.3, 0.2: the third goes first, then the
    second, then the first.  With equal importance the order is least recently
    used."""
    pool = Pool(32, bs)
    cache = Cache(pool, "rsbcm")
    leaves = []
    for i, (score, depth) in enumerate([(0.9, 1), (0.3, 0), (0.8, 3)]):
        toks = [i] * (2 * bs)
        pool.alloc(i, len(toks))
        leaves.append(cache.insert(toks, pool.table(i), score, depth)[0])
        pool.free(i)
    order = [cache.evict(1)[1][0] for _ in range(3)]
    assert order == [leaves[2], leaves[1], leaves[0]], order
    # equal importance: least recently used first
    eq = []
    for i in range(3):
        toks = [10 + i] * bs
        pool.alloc(10 + i, len(toks))
        eq.append(cache.insert(toks, pool.table(10 + i), 0.5, 1)[0])
        pool.free(10 + i)
    cache.match_prefix([10] * bs)
    assert [cache.evict(1)[1][0] for _ in range(3)] == [eq[1], eq[2], eq[0]]
    # a branch score raised on a deep leaf protects its ancestors too
    base = [20] * (2 * bs)
    pool.alloc(20, 4 * bs)
    tbl = pool.table(20)
    n1, _ = cache.insert(base, tbl, 0.1, 0)
    n2, _ = cache.insert(base + [21] * (2 * bs), tbl, 0.1, 2)
    cache.set_score(n2, 3.0)
    assert cache.node_info(n1)[4] == 3.0 and cache.node_info(n2)[4] == 3.0
    pool.free(20)


def run_traces(Cache, Pool, seeds=(0, 1, 2, 3), steps=250, bs=2, num_blocks=40):
    for seed in seeds:
        for policy in ("lru", "rsbcm"):
            rng = np.random.default_rng(1000 + seed)
            pool = Pool(num_blocks, bs, [int(x) for x in rng.permutation(num_blocks)])
            sys = PinnedCache(pool, Cache(pool, policy), bs, policy)
            log = TraceDriver(sys, bs, seed).run(steps)
            kinds = {e[0] for e in log}
            assert {"arrive", "finish", "evict"} <= kinds


def run_radix_pins(Cache, Pool):
    scenario_system_prompt(Cache, Pool, users=200)
    scenario_multi_turn(Cache, Pool)
    scenario_branch_and_backtrack(Cache, Pool)
    scenario_leaf_only_eviction(Cache, Pool)
    scenario_evict_blocks_in_use(Cache, Pool)
    scenario_rsbcm_order(Cache, Pool)
    scenario_batched_admission(Cache, Pool)
    run_traces(Cache, Pool, seeds=(0, 1), steps=200)

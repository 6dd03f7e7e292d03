"""Reference prefix cache over paged KV blocks: a radix tree with locks and leaf
eviction (oracle; test infrastructure only).

Sources:

* "Dismantling the Memory Wall", section "RadixAttention: The Tree of Life for
  Agentic Swarms": the cache is a compressed trie (a node with one child is
  merged into its parent) whose edges hold token runs and the KV locations
  that go with them; finished requests stay in the tree; a new request takes
  the longest cached prefix of its tokens and only computes the rest.  Each
  node carries children, parent, key (tokens), value (KV indices), ``lock_ref``
  and ``last_access_time``.  A request that uses a node raises ``lock_ref`` on
  it and on all its ancestors; when memory runs out, eviction removes least
  recently used leaves whose ``lock_ref`` is 0, so shared prefixes stay.  A
  later turn of a conversation appends to the leaf of the turn before.
* "RKSC - Reasoning-Aware KV Cache Sharing en Confident Early Exit", §2
  "Methodologie", C "RSBCM": under memory pressure blocks go in order of an
  importance omega = branch_score / (depth + 1), lowest first, so deep,
  low-scoring trajectories leave first.

Readings (the pages fix the structure and the policies, not every detail):

* K1  Granularity: the cache holds whole blocks.  A key is cut into runs of
      ``block_size`` tokens; a block matches only when all its tokens match, so
      matches, splits and inserts happen at block boundaries and a partly
      filled last block is never cached.
* K2  ``match_prefix(tokens)`` walks from the root; where the match ends inside
      a node the node is split there (the upper part, a new node, takes the
      matched blocks and the node keeps the rest and its id), so the returned
      node ends exactly at the match.  Every node on the matched path gets the
      current time.  Returns (matched tokens, their block ids, node id); the
      root is id 0.
* K3  Time is a logical clock: one tick per ``match_prefix`` or ``insert``.
      Ties in eviction order go to the smaller node id (the older node).
* K4  ``insert(tokens, blocks, score, depth)`` caches the full blocks of a
      sequence whose block ids are ``blocks`` (its block table).  Where the path
      is cached already the tree keeps its own blocks; the rest becomes one new
      leaf under the last matched node, and the tree takes one pool reference
      on each block it adopts.  Path nodes get the current time and
      score = max(score, their score); a new leaf takes (score, depth).
* K5  ``lock`` / ``unlock`` change ``lock_ref`` by one on the node and every
      ancestor below the root; unlock below zero is an error.
* K6  ``evict(n)`` removes leaves with ``lock_ref`` 0, one at a time, until n
      blocks went back to the free pool or none is left; removing a leaf drops
      the tree's reference on each of its blocks, in key order, and may turn
      its parent into a leaf.  Policy "lru": smallest (last_access_time, id).
      Policy "rsbcm": smallest (score / (depth + 1), last_access_time, id), the
      division in binary64.
* K7  ``set_score(node, s)`` sets the node's score to s and raises every
      ancestor's to at least s (a prefix is worth its best branch).
* K8  A split copies lock_ref, last_access_time, score and depth to the new
      upper node.
* K9  Batched admission, in order: a request matches all but its last token
      (at least one token is computed), locks the match, evicts
      (blocks needed - free blocks) when the pool is short, and starts its
      sequence on the matched blocks; the first request that still does not fit
      is unlocked and stops the batch.  ``finish`` caches each sequence's
      tokens (insert with its score and depth), unlocks its admission node and
      frees the sequence, after checking every entry.
"""

import math

from .pool import RefPool


class RadixError(ValueError):
    """Invalid use of the cache (unknown node, bad argument)."""


class TreeNode:
    def __init__(self, node_id, parent, key, value, tick, score, depth):
        self.id = node_id
        self.children = {}          # first block of the child's key -> child
        self.parent = parent
        self.key = key              # list of blocks, each a tuple of block_size tokens
        self.value = value          # physical block id of each key block
        self.lock_ref = 0
        self.last_access_time = tick
        self.score = float(score)
        self.depth = int(depth)


class RadixCache:
    POLICIES = ("lru", "rsbcm")

    def __init__(self, pool: RefPool, policy: str = "lru"):
        if policy not in self.POLICIES:
            raise RadixError(f"unknown policy {policy!r}")
        self.pool = pool
        self.policy = policy
        self.block_size = pool.block_size
        self.root = TreeNode(0, None, [], [], 0, 0.0, 0)
        self.nodes = {0: self.root}
        self.next_id = 1
        self.clock = 0

    # -- helpers -------------------------------------------------------------
    def _cut(self, tokens):
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        return [tuple(tokens[i * bs:(i + 1) * bs]) for i in range(len(tokens) // bs)]

    @staticmethod
    def _common(a, b):
        n = 0
        while n < len(a) and n < len(b) and a[n] == b[n]:
            n += 1
        return n

    def _split(self, node, m):
        upper = TreeNode(self.next_id, node.parent, node.key[:m], node.value[:m], node.last_access_time,
                         node.score, node.depth)
        self.next_id += 1
        upper.lock_ref = node.lock_ref
        node.parent.children[node.key[0]] = upper
        node.key = node.key[m:]
        node.value = node.value[m:]
        upper.children[node.key[0]] = node
        node.parent = upper
        self.nodes[upper.id] = upper
        return upper

    def _node(self, node_id):
        if node_id not in self.nodes:
            raise KeyError(f"node {node_id} does not exist")
        return self.nodes[node_id]

    def _path(self, node):
        out = []
        while node is not self.root:
            out.append(node)
            node = node.parent
        return out

    # -- K2 ------------------------------------------------------------------
    def match_prefix(self, tokens):
        self.clock += 1
        key = self._cut(tokens)
        node, i, blocks = self.root, 0, []
        while i < len(key) and key[i] in node.children:
            child = node.children[key[i]]
            m = self._common(child.key, key[i:])
            if m < len(child.key):
                child = self._split(child, m)
            child.last_access_time = self.clock
            blocks.extend(child.value)
            i += m
            node = child
        return i * self.block_size, blocks, node.id

    # -- K4 ------------------------------------------------------------------
    def insert(self, tokens, blocks, score=0.0, depth=0):
        key = self._cut(tokens)
        blocks = [int(b) for b in blocks]
        if len(blocks) < len(key):
            raise RadixError("fewer block ids than full blocks")
        if depth < 0:
            raise RadixError("depth must be >= 0")
        if not math.isfinite(score):
            raise RadixError("score must be finite")
        for b in blocks[:len(key)]:
            if not (0 <= b < self.pool.num_blocks) or self.pool.refcount(b) == 0:
                raise RadixError(f"block {b} is not allocated")
        self.clock += 1
        node, i, adopted = self.root, 0, 0
        while i < len(key):
            if key[i] in node.children:
                child = node.children[key[i]]
                m = self._common(child.key, key[i:])
                if m < len(child.key):
                    child = self._split(child, m)
                child.last_access_time = self.clock
                child.score = max(child.score, float(score))
                node = child
                i += m
            else:
                leaf = TreeNode(self.next_id, node, key[i:], blocks[i:len(key)], self.clock, score, depth)
                self.next_id += 1
                for b in leaf.value:
                    self.pool.retain(b)
                node.children[leaf.key[0]] = leaf
                self.nodes[leaf.id] = leaf
                adopted = len(leaf.value)
                node = leaf
                i = len(key)
        return node.id, adopted

    # -- K5 ------------------------------------------------------------------
    def lock(self, node_id):
        for n in self._path(self._node(node_id)):
            n.lock_ref += 1

    def unlock(self, node_id):
        path = self._path(self._node(node_id))
        if any(n.lock_ref == 0 for n in path):
            raise RadixError(f"node {node_id} is not locked")
        for n in path:
            n.lock_ref -= 1

    # -- K7 ------------------------------------------------------------------
    def set_score(self, node_id, score):
        node = self._node(node_id)
        if node is self.root:
            raise RadixError("the root has no score")
        if not math.isfinite(score):
            raise RadixError("score must be finite")
        node.score = float(score)
        for n in self._path(node.parent):
            n.score = max(n.score, float(score))

    # -- K6 ------------------------------------------------------------------
    def priority(self, node):
        if self.policy == "lru":
            return (node.last_access_time, node.id)
        return (node.score / (node.depth + 1), node.last_access_time, node.id)

    def evictable_leaves(self):
        return [n for n in self.nodes.values() if n is not self.root and not n.children and n.lock_ref == 0]

    def evict(self, num_blocks):
        released, evicted = 0, []
        while released < num_blocks:
            leaves = self.evictable_leaves()
            if not leaves:
                break
            victim = min(leaves, key=self.priority)
            for b in victim.value:
                if self.pool.release(b):
                    released += 1
            del victim.parent.children[victim.key[0]]
            del self.nodes[victim.id]
            evicted.append(victim.id)
        return released, evicted

    # -- K9 ------------------------------------------------------------------
    def admit(self, requests, seqs):
        """requests: token lists; returns [(matched tokens, node)] of the admitted prefix."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs) or any(s in self.pool for s in seqs) or any(len(t) < 1 for t in requests):
            raise RadixError("admit: repeated or existing sequence id, or an empty request")
        out = []
        for toks, seq in zip(requests, seqs):
            m, blocks, node = self.match_prefix(list(toks)[:-1])
            self.lock(node)
            need = -(-len(toks) // self.block_size) - len(blocks)
            if need > self.pool.free_count():
                self.evict(need - self.pool.free_count())
            try:
                self.pool.alloc_with_prefix(seq, blocks, len(toks))
            except MemoryError:
                self.unlock(node)
                break
            out.append((m, node))
        return out

    def finish(self, requests, seqs, nodes, scores=None, depths=None):
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise RadixError("finish: repeated sequence id")
        pending = {}
        for i, (toks, seq, node) in enumerate(zip(requests, seqs, nodes)):
            if seq not in self.pool:
                raise KeyError(f"sequence {seq} does not exist")
            if self.pool.is_swapped(seq):
                raise RadixError(f"sequence {seq} is swapped out")
            if len(toks) > self.pool.length(seq):
                raise RadixError("finish: more tokens than the sequence holds")
            for n in self._path(self._node(node)):
                pending[n.id] = pending.get(n.id, 0) + 1
                if pending[n.id] > n.lock_ref:
                    raise RadixError(f"node {node} is not locked")
            if scores is not None and not math.isfinite(scores[i]):
                raise RadixError("score must be finite")
            if depths is not None and depths[i] < 0:
                raise RadixError("depth must be >= 0")
        for i, (toks, seq, node) in enumerate(zip(requests, seqs, nodes)):
            self.insert(toks, self.pool.table(seq), 0.0 if scores is None else scores[i],
                        0 if depths is None else depths[i])
            self.unlock(node)
            self.pool.free(seq)

    def clear(self):
        """Drop every cached node (ids in increasing order, blocks in key order)."""
        for node_id in sorted(self.nodes):
            if node_id == 0:
                continue
            for b in self.nodes[node_id].value:
                self.pool.release(b)
        self.root.children = {}
        self.nodes = {0: self.root}

    # -- queries -------------------------------------------------------------
    def cached_blocks(self):
        return sum(len(n.value) for n in self.nodes.values())

    def evictable_blocks(self):
        return sum(len(n.value) for n in self.nodes.values() if n is not self.root and n.lock_ref == 0)

    def node_ids(self):
        return sorted(self.nodes)

    def node_info(self, node_id):
        """(parent id, block ids, lock_ref, last_access_time, score, depth); parent -1 for the root."""
        n = self._node(node_id)
        return (-1 if n.parent is None else n.parent.id, list(n.value), n.lock_ref, n.last_access_time,
                n.score, n.depth)

    def node_tokens(self, node_id):
        return [t for blk in self._node(node_id).key for t in blk]

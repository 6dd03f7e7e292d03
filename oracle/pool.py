"""Reference block pool with reference counts, fork, copy-on-write append and free
(oracle; test infrastructure only).

Sources:

* "The Reasoning Engine Meltdown", §5 "Paged Memory Management for Dynamic Trees":
  a fork makes the child point at the parent's physical pages without copying
  KV data and raises each shared page's reference count by one; writes go to
  new dedicated pages (copy-on-write); pruning lowers the counts and a page
  whose count reaches 0 returns to the free pool at once.
* Same page, §6 (the ``TreePagedKVCacheManager`` listing): root allocation takes
  ceil(tokens / page_size) pages with count 1 and fails with an out-of-memory
  error *before* changing anything when too few pages are free; fork of an
  unknown parent is a key error; freeing an unknown node does nothing; taking
  a page from an empty pool is an out-of-memory error.
* "Dismantling the Memory Wall", section "PagedAttention ...": token t of a
  sequence is in logical block t // block_size at row t % block_size; only the
  last block is partly filled (at most block_size - 1 wasted slots).  Section
  "Copy-on-Write and Advanced Decoding Strategies": beams share the prompt's
  physical blocks (reference counted) and a branch gets its own block only when
  it diverges.

Readings (the listing's ``append_tokens`` copies no data and only acts on a
capacity overflow, which contradicts the prose; the prose wins):

* R1  The free pool is a FIFO: creation seeds it with ``free_order`` (a
      permutation of the block ids, supplied by the caller), allocation takes
      from the front, a freed block goes to the back.  (The listing's ``set.pop``
      order is unspecified; fixing one order makes indices comparable exactly.)
* R2  ``alloc(seq, n)`` takes ceil(n / block_size) blocks with count 1, or raises
      MemoryError with nothing changed.
* R3  ``fork(parent, child)``: the child's table is a copy of the parent's,
      including a partly filled last block; every block's count goes up by one.
* R4  ``plan_append(seqs)`` appends one token to each sequence, in batch order:
      pos = len, j = pos // block_size, off = pos % block_size.
        - off == 0: a new block is allocated and appended to the table.
        - off > 0 and count(table[j]) > 1: a new block Y is allocated, rows
          [0, off) of X = table[j] are copied to Y, count(X) drops by one and
          table[j] = Y (copy-on-write of a shared, partly filled block).
        - slot = table[j] * block_size + off; len += 1.
      The whole batch either fits in the free pool or raises MemoryError with
      nothing changed.
* R5  ``free(seq)`` lowers the counts in table order; a block reaching 0 goes to
      the back of the free pool.  An unknown sequence is a no-op.
* R6  Holders other than sequences (a prefix cache) take and drop references
      with ``retain`` / ``release``; ``alloc_with_prefix(seq, prefix, n)`` starts a
      sequence on cached blocks ("Dismantling the Memory Wall", "RadixAttention":
      a request that shares a cached prefix points at the existing memory and
      only computes the new tokens): its table is ``prefix`` (one more reference
      each) followed by fresh blocks for the rest of the n tokens, or MemoryError
      with nothing changed.
* R7  Swap space ("Dismantling the Memory Wall", "Cross-Tier Memory Offloading":
      when the KV cache overflows the GPU, blocks move down to CPU memory and
      are brought back before attention needs them).  The pool also keeps
      ``num_host_slots`` host slots with their own FIFO free list (seeded by
      ``host_order``).  ``swap_out(seq)`` moves, in table order, every block that
      the sequence holds alone (count 1) to a host slot taken from the front of
      the host list, and returns that device block to the back of the device
      list; blocks shared with other holders stay on the device and keep the
      sequence's reference.  ``swap_in(seq)`` takes a device block from the
      front of the device list for each host-resident entry, in table order,
      and returns the host slot to the back of the host list.  Both are
      all-or-nothing (MemoryError with nothing changed) and return the copies to
      perform: (device block, host slot) pairs out, (host slot, device block)
      pairs in.  A swapped-out sequence cannot be appended to, forked or
      exported; freeing it releases its host slots (table order) and its
      remaining device references.
"""

from collections import deque

import numpy as np


class RefPoolError(ValueError):
    """Invalid use of the pool (duplicate id, bad argument)."""


class RefPool:
    def __init__(self, num_blocks: int, block_size: int, free_order=None, num_host_slots: int = 0,
                 host_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise RefPoolError("num_blocks must be >= 0 and block_size > 0")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(self.num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise RefPoolError("free_order must be a permutation of range(num_blocks)")
        self._free = deque(order)
        self._ref = [0] * self.num_blocks
        self._tables = {}
        self._lens = {}
        self.num_host_slots = int(num_host_slots)
        horder = list(range(self.num_host_slots)) if host_order is None else [int(x) for x in host_order]
        if sorted(horder) != list(range(self.num_host_slots)):
            raise RefPoolError("host_order must be a permutation of range(num_host_slots)")
        self._host_free = deque(horder)
        self._swapped = {}   # seq -> [("host", slot) | ("device", block)] in table order

    # -- queries -----------------------------------------------------------
    def table(self, seq):
        if seq in self._swapped:
            raise RefPoolError(f"sequence {seq!r} is swapped out")
        return list(self._tables[seq])

    def length(self, seq):
        return self._lens[seq]

    def refcount(self, block: int) -> int:
        return self._ref[block]

    def free_count(self) -> int:
        return len(self._free)

    def free_list(self):
        return list(self._free)

    def sequences(self):
        return list(self._tables.keys())

    def __contains__(self, seq):
        return seq in self._tables or seq in self._swapped

    def is_swapped(self, seq):
        return seq in self._swapped

    def host_free_count(self) -> int:
        return len(self._host_free)

    def host_free_list(self):
        return list(self._host_free)

    def placement(self, seq):
        """Table entries of a sequence as ("device", block) / ("host", slot)."""
        if seq in self._swapped:
            return list(self._swapped[seq])
        return [("device", b) for b in self._tables[seq]]

    # -- R2 ----------------------------------------------------------------
    def alloc(self, seq, num_tokens: int):
        if seq in self:
            raise RefPoolError(f"sequence {seq!r} already exists")
        if num_tokens < 0:
            raise RefPoolError("num_tokens must be >= 0")
        need = -(-int(num_tokens) // self.block_size)
        if need > len(self._free):
            raise MemoryError(f"OOM: requested {need} blocks, only {len(self._free)} free")
        blocks = []
        for _ in range(need):
            b = self._free.popleft()
            self._ref[b] = 1
            blocks.append(b)
        self._tables[seq] = blocks
        self._lens[seq] = int(num_tokens)
        return list(blocks)

    # -- R3 ----------------------------------------------------------------
    def fork(self, parent, child):
        if parent in self._swapped:
            raise RefPoolError(f"parent {parent!r} is swapped out")
        if parent not in self._tables:
            raise KeyError(f"parent {parent!r} does not exist")
        if child in self:
            raise RefPoolError(f"sequence {child!r} already exists")
        for b in self._tables[parent]:
            self._ref[b] += 1
        self._tables[child] = list(self._tables[parent])
        self._lens[child] = self._lens[parent]
        return list(self._tables[child])

    # -- R5 ----------------------------------------------------------------
    def free(self, seq):
        if seq in self._swapped:
            for kind, x in self._swapped.pop(seq):
                if kind == "host":
                    self._host_free.append(x)
                else:
                    self._ref[x] -= 1
                    if self._ref[x] == 0:
                        self._free.append(x)
            del self._lens[seq]
            return
        if seq not in self._tables:
            return
        for b in self._tables[seq]:
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._free.append(b)
        del self._tables[seq]
        del self._lens[seq]

    # -- R6 ----------------------------------------------------------------
    def retain(self, block: int):
        if not (0 <= block < self.num_blocks) or self._ref[block] == 0:
            raise RefPoolError(f"block {block} is not allocated")
        self._ref[block] += 1

    def release(self, block: int) -> bool:
        """Drop one reference; True when the block went back to the free pool."""
        if not (0 <= block < self.num_blocks) or self._ref[block] == 0:
            raise RefPoolError(f"block {block} is not allocated")
        self._ref[block] -= 1
        if self._ref[block] == 0:
            self._free.append(block)
            return True
        return False

    def alloc_with_prefix(self, seq, prefix_blocks, num_tokens: int):
        prefix_blocks = [int(b) for b in prefix_blocks]
        if seq in self:
            raise RefPoolError(f"sequence {seq!r} already exists")
        if num_tokens < len(prefix_blocks) * self.block_size:
            raise RefPoolError("num_tokens must cover the prefix blocks")
        for b in prefix_blocks:
            if not (0 <= b < self.num_blocks) or self._ref[b] == 0:
                raise RefPoolError(f"prefix block {b} is not allocated")
        need = -(-int(num_tokens) // self.block_size) - len(prefix_blocks)
        if need > len(self._free):
            raise MemoryError(f"OOM: requested {need} blocks, only {len(self._free)} free")
        for b in prefix_blocks:
            self._ref[b] += 1
        blocks = list(prefix_blocks)
        for _ in range(need):
            b = self._free.popleft()
            self._ref[b] = 1
            blocks.append(b)
        self._tables[seq] = blocks
        self._lens[seq] = int(num_tokens)
        return list(blocks)

    # -- R7 ----------------------------------------------------------------
    def swap_out(self, seq):
        if seq in self._swapped:
            raise RefPoolError(f"sequence {seq!r} is already swapped out")
        if seq not in self._tables:
            raise KeyError(f"sequence {seq!r} does not exist")
        table = self._tables[seq]
        alone = [b for b in table if self._ref[b] == 1]
        if len(alone) > len(self._host_free):
            raise MemoryError(f"OOM: {len(alone)} host slots needed, {len(self._host_free)} free")
        entries, copies = [], []
        for b in table:
            if self._ref[b] == 1:
                h = self._host_free.popleft()
                copies.append((b, h))
                entries.append(("host", h))
                self._ref[b] = 0
                self._free.append(b)
            else:
                entries.append(("device", b))
        del self._tables[seq]
        self._swapped[seq] = entries
        return copies

    def swap_in(self, seq):
        if seq not in self._swapped:
            if seq in self._tables:
                raise RefPoolError(f"sequence {seq!r} is not swapped out")
            raise KeyError(f"sequence {seq!r} does not exist")
        entries = self._swapped[seq]
        need = sum(1 for kind, _ in entries if kind == "host")
        if need > len(self._free):
            raise MemoryError(f"OOM: {need} device blocks needed, {len(self._free)} free")
        table, copies = [], []
        for kind, x in entries:
            if kind == "host":
                y = self._free.popleft()
                self._ref[y] = 1
                copies.append((x, y))
                self._host_free.append(x)
                table.append(y)
            else:
                table.append(x)
        del self._swapped[seq]
        self._tables[seq] = table
        return copies

    # -- R4 ----------------------------------------------------------------
    def plan_append(self, seqs):
        """Append one token to each sequence in ``seqs`` (batch order).

        Returns (slots, cows): slots[i] is the flat slot of seqs[i]'s new token,
        cows is a list of (src_block, dst_block, rows) copies to perform first.
        """
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise RefPoolError("a sequence may appear at most once per append batch")
        for s in seqs:
            if s in self._swapped:
                raise RefPoolError(f"sequence {s!r} is swapped out")
            if s not in self._tables:
                raise KeyError(f"sequence {s!r} does not exist")
        # capacity for the whole batch first (all-or-nothing)
        need = 0
        taken = {}
        for s in seqs:
            pos = self._lens[s]
            j, off = divmod(pos, self.block_size)
            if off == 0:
                need += 1
            else:
                x = self._tables[s][j]
                if self._ref[x] + taken.get(x, 0) > 1:
                    need += 1
                    taken[x] = taken.get(x, 0) - 1
        if need > len(self._free):
            raise MemoryError(f"OOM: append batch needs {need} blocks, only {len(self._free)} free")
        slots = []
        cows = []
        for s in seqs:
            table = self._tables[s]
            pos = self._lens[s]
            j, off = divmod(pos, self.block_size)
            if off == 0:
                assert len(table) == j
                y = self._free.popleft()
                self._ref[y] = 1
                table.append(y)
            else:
                x = table[j]
                if self._ref[x] > 1:
                    y = self._free.popleft()
                    self._ref[y] = 1
                    cows.append((x, y, off))
                    self._ref[x] -= 1
                    table[j] = y
            slots.append(table[j] * self.block_size + off)
            self._lens[s] = pos + 1
        return slots, cows

    # -- export ------------------------------------------------------------
    def export_tables(self, seqs, max_blocks: int, pad: int = -1):
        seqs = list(seqs)
        bt = np.full((len(seqs), max_blocks), pad, dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        for i, s in enumerate(seqs):
            if s in self._swapped:
                raise RefPoolError(f"sequence {s!r} is swapped out")
            t = self._tables[s]
            if len(t) > max_blocks:
                raise RefPoolError(f"sequence {s!r} has {len(t)} blocks > max_blocks {max_blocks}")
            bt[i, : len(t)] = t
            lens[i] = self._lens[s]
        return bt, lens


def apply_append(k_pages, v_pages, slots, cows, k_new, v_new):
    """Perform a planned append on copies of the pages and return them.

    First every copy-on-write (rows [0, rows) of block src into block dst, for K
    and V), then every token write: flat slot ``slot`` is block slot // block_size,
    row slot % block_size.  Negative slots are skipped (padding).
    """
    k = np.array(k_pages, copy=True)
    v = np.array(v_pages, copy=True)
    block_size = k.shape[1]
    for src, dst, rows in cows:
        k[dst, :rows] = k[src, :rows]
        v[dst, :rows] = v[src, :rows]
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    for i, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        blk, row = divmod(slot, block_size)
        k[blk, row] = k_new[i]
        v[blk, row] = v_new[i]
    return k, v


def apply_swap(dst_pages, src_pages, copies):
    """Copy whole blocks: dst_pages[d] = src_pages[s] for each (s, d) in ``copies``
    (device -> host for ``swap_out``'s (block, slot) pairs, host -> device for
    ``swap_in``'s (slot, block) pairs).  Returns a new array."""
    out = np.array(dst_pages, copy=True)
    for s, d in copies:
        out[d] = src_pages[s]
    return out

"""Seeded synthetic inputs for the paged decode-attention tests, bench and smoke run.

This module is shared by the oracle side and the HIP side of every test.  It
holds none of the method's arithmetic: it draws random numbers, fixes shapes,
and writes down *what happens to the sequences* (allocate, fork, append, free)
as a script of operations.  Each side replays the script on its own block pool
(the oracle's ``RefPool`` or the library's C++ pool), so block tables, slots and
copy-on-write decisions are computed independently on the two sides.

Every physical block of the pool starts out holding random K/V values, so a
sequence's cached tokens are simply whatever its table points at; only tokens
appended through ``kv_append`` get new, separately drawn values.

Workloads (seed = workload number, structure drawn from one numpy PCG64
generator in the order lengths -> tree -> placement permutation; q, k, v and
new tokens from seeded torch generators on the target device):

1. tiny tree: 4 branches share a 256-token prefix, 32-token private suffixes;
   Hq = Hkv = 8, d = 64, fp16.
2. Llama-3-8B-shaped decode layer: 64 independent sequences, lengths uniform
   in [512, 4096]; Hq = 32, Hkv = 8, d = 128, bf16.
3. tree search: 16 problems x 64 branches, 2048-token prefix per problem,
   suffix lengths geometric with mean 256 clipped to [64, 1024]; GQA 32/8,
   d = 128, bf16.
4. 70B-MHA-shaped layer: 16 sequences x 8192 tokens, Hq = Hkv = 64, d = 128,
   fp16 (2^32 bytes of K+V).
5. radix tree with backtracking: 4096-token root, branching 4, depth 4
   (256 leaves), 256 tokens per level; 16 decode steps, each appending one
   token per leaf; after steps 3, 7, 11 and 15 the 64 lowest-scoring leaves
   are pruned and 64 survivors are forked into their places, so the next
   append hits shared, partly filled tail blocks; GQA 32/8, d = 128, bf16.

Request traces for the prefix cache (token ids only):

* ``system_prompt_requests``: many users whose requests all begin with one
  long system prompt (1,000 users and a 2,000-token prompt in the RadixAttention
  section's example), each followed by the user's own tokens.
* ``agent_sessions``: multi-turn sessions over a few shared system prompts;
  each turn resends the session's whole history plus new tokens, and sessions
  fork (two continuations of one history, as an agent exploring branches).

Values are N(0, 1) in fp32, rounded to nearest-even fp16/bf16.  Physical
placement is a seeded permutation of the pool (the pool's initial free list).
The pool is the blocks a workload needs plus 25 %.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16


@dataclasses.dataclass
class Step:
    """One decode step: append one token to each of ``append_rows`` (batch
    order), then decode ``decode_rows``; afterwards replay ``after_ops``."""

    append_rows: List[int]
    decode_rows: List[int]
    after_ops: list


@dataclasses.dataclass
class Workload:
    number: int
    name: str
    description: str
    dtype: str  # "f16" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray  # int32 permutation of range(num_blocks)
    build_ops: list  # script replayed on a pool before the first step
    steps: List[Step]
    max_blocks: int  # block-table width
    seed: int
    logical_tokens: int = 0  # tokens summed over decode rows at step 0 (each branch counted)
    unique_tokens: int = 0  # distinct tokens referenced at step 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def batch(self) -> int:
        return len(self.steps[0].decode_rows)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def bytes_per_token(self) -> int:
        """K plus V bytes of one token for all KV heads of the layer."""
        return 2 * self.num_kv_heads * self.head_dim * 2


# ---------------------------------------------------------------------------
# script replay (dispatch only)


def replay(pool, ops, allow_cow: bool = False) -> int:
    """Replay a script of pool operations on ``pool`` (RefPool or the library's
    BlockPool; both expose alloc / fork / free / plan_append).

    ("alloc", seq, n) | ("fork", parent, child) | ("free", seq) |
    ("extend", seqs, counts): append counts[i] tokens to seqs[i], one token per
    sequence per batch, batches in order, until every count is used up.  The
    five named workloads never hit a partly filled shared block while building,
    so their appends make no copies (asserted unless ``allow_cow``).  Build
    appends move no data: the blocks already hold random values.  Returns the
    number of copy-on-write events seen.
    """
    n_cow = 0
    for op in ops:
        kind = op[0]
        if kind == "alloc":
            pool.alloc(op[1], op[2])
        elif kind == "fork":
            pool.fork(op[1], op[2])
        elif kind == "free":
            pool.free(op[1])
        elif kind == "extend":
            seqs, counts = list(op[1]), list(op[2])
            for r in range(max(counts) if counts else 0):
                batch = [s for s, c in zip(seqs, counts) if c > r]
                _, cows = pool.plan_append(batch)
                n_cow += len(cows)
                assert allow_cow or len(cows) == 0, "build scripts must not copy blocks"
        else:
            raise ValueError(f"unknown op {kind!r}")
    return n_cow


# ---------------------------------------------------------------------------
# data generators


def _torch():
    import torch

    return torch


def _normal_bits(shape, dtype: str, seed: int, device) -> "object":
    """N(0,1) fp32 draws rounded to fp16/bf16, returned as an int16 tensor of bits."""
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    out = torch.empty(shape, dtype=tdt, device=device)
    flat = out.view(-1)
    chunk = 1 << 26
    for i in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - i)
        flat[i : i + n] = torch.randn(n, generator=gen, device=device, dtype=torch.float32).to(tdt)
    return out.view(torch.int16)


def make_pages(w: Workload, device="cpu"):
    """(k_pages, v_pages) as int16 bit tensors [num_blocks, block_size, Hkv, d]."""
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    k = _normal_bits(shape, w.dtype, w.seed * 1000 + 2, device)
    v = _normal_bits(shape, w.dtype, w.seed * 1000 + 3, device)
    return k, v


def make_fp8_pages(w: Workload, device="cpu"):
    """FP8 pages for a workload: random E4M3 codes of magnitude 2^-2 .. 2^5 with random signs,
    and per-(block, head, row) power-of-two scales 2^-5 or 2^-4 (elements of magnitude about
    2^-7 .. 2^1, like quantized N(0, 1) data).  Returns (k_codes, v_codes, k_scales, v_scales)
    as uint8 [num_blocks, block_size, Hkv, d] and float32 [num_blocks, Hkv, block_size]."""
    torch = _torch()
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed) * 7 + 3)
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    out = []
    for _ in range(2):
        mag = torch.randint(0x28, 0x61, shape, generator=gen, device=device, dtype=torch.int32)
        sign = torch.randint(0, 2, shape, generator=gen, device=device, dtype=torch.int32) * 0x80
        out.append((mag | sign).to(torch.uint8))
    for _ in range(2):
        e = torch.randint(-5, -3, (w.num_blocks, w.num_kv_heads, w.block_size), generator=gen, device=device)
        out.append(torch.exp2(e.to(torch.float32)))
    return tuple(out)


def make_q(w: Workload, step: int = 0, device="cpu"):
    """Queries for step ``step`` as an int16 bit tensor [B, Hq, d]."""
    return _normal_bits((len(w.steps[step].decode_rows), w.num_q_heads, w.head_dim), w.dtype,
                        w.seed * 1000 + 1 + 10 * step, device)


def make_new_tokens(w: Workload, step: int = 0, device="cpu"):
    """(k_new, v_new) for the appends of step ``step``: int16 bits [N, Hkv, d]."""
    n = len(w.steps[step].append_rows)
    shape = (n, w.num_kv_heads, w.head_dim)
    return (_normal_bits(shape, w.dtype, w.seed * 1000 + 4 + 10 * step, device),
            _normal_bits(shape, w.dtype, w.seed * 1000 + 5 + 10 * step, device))


def _pool_size(needed_blocks: int) -> int:
    return int(math.ceil(needed_blocks * 1.25))


def _blocks(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-n_tokens // block_size)


# ---------------------------------------------------------------------------
# the five workloads


def tiny_tree(seed: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    prefix, suffix, branches = 256, 32, 4
    needed = _blocks(prefix) + branches * _blocks(suffix)
    nblk = _pool_size(needed)
    free_order = rng.permutation(nblk).astype(np.int32)
    root = 1000
    rows = list(range(branches))
    ops = [("alloc", root, prefix)]
    ops += [("fork", root, r) for r in rows]
    ops += [("free", root)]
    ops += [("extend", rows, [suffix - 1] * branches)]
    total = prefix + suffix
    return Workload(1, "tiny_tree", "4 branches x (256 shared + 32 private) tokens, Hq=Hkv=8, d=64, fp16",
                    "f16", 8, 8, 64, BLOCK_SIZE, nblk, free_order, ops, [Step(rows, rows, [])],
                    max_blocks=_blocks(total), seed=seed,
                    logical_tokens=branches * total, unique_tokens=prefix + branches * suffix)


def llama8b_decode(seed: int = 2, batch: int = 64, lo: int = 512, hi: int = 4096) -> Workload:
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi + 1, size=batch)
    needed = int(sum(_blocks(int(n)) for n in lens))
    nblk = _pool_size(needed)
    free_order = rng.permutation(nblk).astype(np.int32)
    rows = list(range(batch))
    ops = [("alloc", r, int(lens[r]) - 1) for r in rows]
    return Workload(2, "llama8b_decode",
                    f"{batch} sequences, lengths U[{lo},{hi}], Hq=32, Hkv=8, d=128, bf16, no sharing",
                    "bf16", 32, 8, 128, BLOCK_SIZE, nblk, free_order, ops, [Step(rows, rows, [])],
                    max_blocks=_blocks(hi), seed=seed,
                    logical_tokens=int(lens.sum()), unique_tokens=int(lens.sum()))


def tree_search(seed: int = 3, problems: int = 16, branches: int = 64, prefix: int = 2048) -> Workload:
    rng = np.random.default_rng(seed)
    suffix = np.clip(rng.geometric(1.0 / 256.0, size=problems * branches), 64, 1024)
    needed = problems * _blocks(prefix) + int(sum(_blocks(int(s)) for s in suffix))
    nblk = _pool_size(needed)
    free_order = rng.permutation(nblk).astype(np.int32)
    ops = []
    rows = []
    for p in range(problems):
        root = 100000 + p
        mine = [p * branches + i for i in range(branches)]
        ops.append(("alloc", root, prefix))
        ops += [("fork", root, r) for r in mine]
        ops.append(("free", root))
        rows += mine
    ops.append(("extend", rows, [int(s) - 1 for s in suffix]))
    lens = prefix + suffix
    return Workload(3, "tree_search",
                    f"{problems} problems x {branches} branches, {prefix}-token shared prefix, "
                    "suffix geometric(mean 256) clipped [64,1024], Hq=32, Hkv=8, d=128, bf16",
                    "bf16", 32, 8, 128, BLOCK_SIZE, nblk, free_order, ops, [Step(rows, rows, [])],
                    max_blocks=_blocks(prefix + 1024), seed=seed,
                    logical_tokens=int(lens.sum()), unique_tokens=problems * prefix + int(suffix.sum()))


def mha70b_layer(seed: int = 4, batch: int = 16, length: int = 8192) -> Workload:
    rng = np.random.default_rng(seed)
    needed = batch * _blocks(length)
    nblk = _pool_size(needed)
    free_order = rng.permutation(nblk).astype(np.int32)
    rows = list(range(batch))
    ops = [("alloc", r, length - 1) for r in rows]
    return Workload(4, "mha70b_layer", f"{batch} x {length} tokens, Hq=Hkv=64, d=128, fp16",
                    "f16", 64, 64, 128, BLOCK_SIZE, nblk, free_order, ops, [Step(rows, rows, [])],
                    max_blocks=_blocks(length), seed=seed,
                    logical_tokens=batch * length, unique_tokens=batch * length)


def radix_backtrack(seed: int = 5, root_tokens: int = 4096, branching: int = 4, depth: int = 4,
                    level_tokens: int = 256, steps: int = 16, prune: int = 64) -> Workload:
    rng = np.random.default_rng(seed)
    n_nodes = 1 + sum(branching ** k for k in range(1, depth + 1))
    unique = root_tokens + sum(branching ** k for k in range(1, depth + 1)) * level_tokens
    needed = _blocks(unique)
    nblk = _pool_size(needed)
    # tree first (it is fixed: node ids in breadth-first order), then placement
    free_order = rng.permutation(nblk).astype(np.int32)
    ops = [("alloc", 0, root_tokens)]
    level = [0]
    next_id = 1
    for _ in range(depth):
        children = []
        for parent in level:
            for _ in range(branching):
                ops.append(("fork", parent, next_id))
                children.append(next_id)
                next_id += 1
        ops.append(("extend", children, [level_tokens] * len(children)))
        level = children
    assert next_id == n_nodes
    leaves = list(level)
    step_list = []
    for s in range(1, steps + 1):
        rows = list(leaves)
        after = []
        if s % 4 == 3 and prune > 0:
            scores = rng.random(len(leaves))
            order = np.argsort(scores, kind="stable")
            pruned = sorted(int(i) for i in order[:prune])
            survivors = sorted(int(i) for i in order[prune:])
            picks = rng.choice(survivors, size=prune, replace=False)
            after += [("free", leaves[i]) for i in pruned]
            for slot, p in zip(pruned, picks):
                after.append(("fork", leaves[int(p)], next_id))
                leaves[slot] = next_id
                next_id += 1
        step_list.append(Step(rows, rows, after))
    leaf_len = root_tokens + depth * level_tokens
    return Workload(5, "radix_backtrack",
                    f"root {root_tokens} tokens, branching {branching}, depth {depth} ({len(leaves)} leaves), "
                    f"{level_tokens} tokens per level, {steps} append+decode steps with backtracking, "
                    "Hq=32, Hkv=8, d=128, bf16",
                    "bf16", 32, 8, 128, BLOCK_SIZE, nblk, free_order, ops, step_list,
                    max_blocks=_blocks(leaf_len + steps), seed=seed,
                    logical_tokens=len(leaves) * leaf_len, unique_tokens=unique)


def chunked_prefill(seed: int = 6, cached: int = 28672, slice_tokens: int = 4096) -> Workload:
    """One Llama-3-8B-shaped sequence in the middle of a chunked prefill: the last
    4,096-token slice of a 32,768-token prompt ("Dismantling the Memory Wall",
    "Chunked Prefill": a 32,000-token prompt processed under a 4,096-token budget)
    attends causally to the 28,672 tokens cached before it and to itself."""
    rng = np.random.default_rng(seed)
    total = cached + slice_tokens
    nblk = _pool_size(_blocks(total))
    free_order = rng.permutation(nblk).astype(np.int32)
    ops = [("alloc", 0, total)]
    return Workload(6, "chunked_prefill",
                    f"1 sequence, {slice_tokens}-token slice over {cached} cached tokens, Hq=32, Hkv=8, d=128, bf16",
                    "bf16", 32, 8, 128, BLOCK_SIZE, nblk, free_order, ops, [Step([], [0], [])],
                    max_blocks=_blocks(total), seed=seed, logical_tokens=total, unique_tokens=total)


# Query tokens per decode row for the multi-token (extend) measurements: the
# verify pass scores the last 8 tokens of every tree-search branch; the chunked
# prefill scores its whole slice.
EXTEND_QUERY_TOKENS = {3: 8, 6: 4096}


WORKLOADS = {
    1: tiny_tree,
    2: llama8b_decode,
    3: tree_search,
    4: mha70b_layer,
    5: radix_backtrack,
    6: chunked_prefill,
}


def get(number: int, **kw) -> Workload:
    return WORKLOADS[int(number)](**kw)


# ---------------------------------------------------------------------------
# small random cases for parity sweeps (shapes only; still no method arithmetic)


def random_forest(seed: int, num_rows: int, max_len: int, dtype: str, num_q_heads: int, num_kv_heads: int,
                  head_dim: int, share_prob: float = 0.5, min_len: int = 0) -> Workload:
    """Random small workload: some rows are forks of earlier rows (sharing their
    blocks, sometimes at unaligned lengths), lengths include 0, 1 and ragged
    tails.  Used by the parity sweeps at sizes the oracle finishes quickly."""
    rng = np.random.default_rng(seed)
    ops = []
    lens = {}
    rows = []
    next_id = 0
    for _ in range(num_rows):
        if rows and rng.random() < share_prob:
            parent = rows[int(rng.integers(0, len(rows)))]
            child = next_id
            next_id += 1
            ops.append(("fork", parent, child))
            extra = int(rng.integers(0, max(1, max_len - lens[parent])))
            lens[child] = lens[parent] + extra
            if extra:
                ops.append(("extend", [child], [extra]))
            rows.append(child)
        else:
            n = int(rng.integers(min_len, max_len + 1))
            ops.append(("alloc", next_id, n))
            lens[next_id] = n
            rows.append(next_id)
            next_id += 1
    needed = sum(_blocks(lens[r]) + 1 for r in rows) + 4
    nblk = _pool_size(needed)
    free_order = rng.permutation(nblk).astype(np.int32)
    logical = sum(lens[r] for r in rows)
    return Workload(0, f"random_forest_{seed}", "random small forest", dtype, num_q_heads, num_kv_heads,
                    head_dim, BLOCK_SIZE, nblk, free_order, ops, [Step([], rows, [])],
                    max_blocks=_blocks(max_len) + 1, seed=seed, logical_tokens=logical, unique_tokens=0)


# ---------------------------------------------------------------------------
# request traces for the prefix cache


def system_prompt_requests(seed: int = 7, users: int = 1000, prompt_tokens: int = 2000, user_lo: int = 1,
                           user_hi: int = 256, vocab: int = 32000) -> List[np.ndarray]:
    """Token lists (int32) of ``users`` requests: one shared ``prompt_tokens``-token
    system prompt, then the user's own tokens (length uniform in [user_lo, user_hi])."""
    rng = np.random.default_rng(seed)
    prompt = rng.integers(0, vocab, size=prompt_tokens)
    lens = rng.integers(user_lo, user_hi + 1, size=users)
    return [np.concatenate([prompt, rng.integers(0, vocab, size=int(n))]).astype(np.int32) for n in lens]


def agent_sessions(seed: int = 8, requests: int = 2000, prompts: int = 8, prompt_lo: int = 512,
                   prompt_hi: int = 2048, msg_lo: int = 16, msg_hi: int = 256, open_max: int = 64,
                   fork_p: float = 0.2, vocab: int = 32000, meta: bool = False):
    """Token lists of a multi-turn, branching request stream.  Each request is, with
    equal odds while fewer than ``open_max`` sessions are open, a new session (one of
    ``prompts`` system prompts plus a message) or the next turn of a random open
    session (its history plus a reply and a message, uniform in [msg_lo, msg_hi]
    tokens each); a turn forks its session with probability ``fork_p`` (the old
    history stays open as a second branch).  With ``meta``, also returns per
    request (branch score, depth): the depth is the turn number within the
    session's branch, the score a uniform [0, 1) draw per branch."""
    rng = np.random.default_rng(seed)
    sys_prompts = [rng.integers(0, vocab, size=int(rng.integers(prompt_lo, prompt_hi + 1))) for _ in range(prompts)]
    sessions: List[list] = []   # [tokens, depth, score]
    out, info = [], []
    for _ in range(requests):
        if not sessions or (len(sessions) < open_max and rng.random() < 0.5):
            toks = np.concatenate([sys_prompts[int(rng.integers(prompts))],
                                   rng.integers(0, vocab, size=int(rng.integers(msg_lo, msg_hi + 1)))])
            sessions.append([toks, 0, float(rng.random())])
            depth, score = 0, sessions[-1][2]
        else:
            i = int(rng.integers(len(sessions)))
            toks = np.concatenate([sessions[i][0],
                                   rng.integers(0, vocab, size=int(rng.integers(2 * msg_lo, 2 * msg_hi + 1)))])
            depth = sessions[i][1] + 1
            if rng.random() < fork_p:
                sessions.append([toks, depth, float(rng.random())])
                score = sessions[-1][2]
            else:
                sessions[i][0], sessions[i][1] = toks, depth
                score = sessions[i][2]
        out.append(toks.astype(np.int32))
        info.append((score, depth))
    return (out, info) if meta else out

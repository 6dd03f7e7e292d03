"""Block tables that the prefix cache hands out, fed to the device path.

Requests reuse cached prefix blocks (no K/V written for the matched tokens),
write only their new tokens with ``kv_append``, and decode through the tables;
the oracle reads each request's *logical* K/V from a host record of what was
written for it (or for the request whose blocks it matched), not from the
device pages, so a block that eviction handed out while still in use and that
was overwritten would show up as a mismatch."""

import numpy as np
import pytest

import workloads
from gpu_util import ATOL, bits_np, max_err, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HQ, HKV, D, BS = 32, 8, 128, 16


@pytest.fixture(scope="module")
def pkv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_21_amd as m

    return m


def _bits(gen, shape):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)


class Harness:
    def __init__(self, pk, num_blocks, policy="lru", seed=0):
        self.pk = pk
        order = np.random.default_rng(seed).permutation(num_blocks).astype(np.int32)
        self.pool = pk.BlockPool(num_blocks, BS, order)
        self.cache = pk.RadixCache(self.pool, policy)
        gen = torch.Generator().manual_seed(seed)
        # stale contents everywhere: only written rows may ever be read
        self.k = _bits(gen, (num_blocks, BS, HKV, D)).cuda()
        self.v = _bits(gen, (num_blocks, BS, HKV, D)).cuda()
        self.gen = gen
        self.logical = {}       # seq -> (k bits [n, Hkv, d], v bits) as a host record
        self.block_data = {}    # block id -> (k rows, v rows) recorded when the block was filled
        self.locked = {}
        self.evictions = 0

    def admit(self, seq, toks):
        m, blocks, node = self.cache.match_prefix(toks[:-1])
        self.cache.lock(node)
        try:
            self.pool.alloc_with_prefix(seq, blocks, len(toks))
        except MemoryError:
            need = -(-len(toks) // BS) - len(blocks)
            self.cache.evict(need)
            self.evictions += 1
            self.pool.alloc_with_prefix(seq, blocks, len(toks))
        self.locked[seq] = node
        table = self.pool.table(seq)
        n_new = len(toks) - m
        k_new = _bits(self.gen, (n_new, HKV, D))
        v_new = _bits(self.gen, (n_new, HKV, D))
        pos = np.arange(m, len(toks))
        slots = np.asarray(table, dtype=np.int64)[pos // BS] * BS + pos % BS
        self.pk.kv_append(self.k, self.v, k_new.cuda(), v_new.cuda(), torch.from_numpy(slots).cuda(), dtype="bf16")
        # logical record: matched blocks as recorded when they were filled, then the new rows
        kk = [self.block_data[b][0] for b in blocks] + [k_new.numpy().view(np.uint16)]
        vv = [self.block_data[b][1] for b in blocks] + [v_new.numpy().view(np.uint16)]
        self.logical[seq] = (np.concatenate(kk), np.concatenate(vv))
        for j in range(m // BS, len(toks) // BS):   # blocks this request filled
            self.block_data[table[j]] = (self.logical[seq][0][j * BS:(j + 1) * BS],
                                         self.logical[seq][1][j * BS:(j + 1) * BS])
        return m

    def finish(self, seq, toks):
        self.cache.insert(toks, self.pool.table(seq))
        self.cache.unlock(self.locked.pop(seq))
        self.pool.free(seq)
        del self.logical[seq]

    def decode_and_check(self, seqs, plan=False):
        import oracle

        bt, lens = self.pool.export_tables(seqs, max(len(self.pool.table(s)) for s in seqs))
        q = _bits(self.gen, (len(seqs), HQ, D))
        scale = 1.0 / np.sqrt(D)
        cplan = self.pk.CascadePlan(bt, lens, HQ, HKV, BS) if plan else None
        if cplan is not None:
            cplan.upload(device="cuda")
        out = self.pk.paged_decode_attn(q.cuda(), self.k, self.v, torch.from_numpy(bt).cuda(),
                                        torch.from_numpy(lens).cuda(), int(lens.max()), scale=scale, plan=cplan,
                                        dtype="bf16")
        torch.cuda.synchronize()
        # oracle on the logical records, laid out contiguously
        nb = [-(-int(n) // BS) for n in lens]
        kp = np.zeros((sum(nb), BS, HKV, D), dtype=np.uint16)
        vp = np.zeros_like(kp)
        obt = np.full((len(seqs), max(nb)), -1, dtype=np.int32)
        off = 0
        for i, s in enumerate(seqs):
            k, v = self.logical[s]
            n = k.shape[0]
            kp.reshape(-1, HKV, D)[off * BS:off * BS + n] = k
            vp.reshape(-1, HKV, D)[off * BS:off * BS + n] = v
            obt[i, :nb[i]] = np.arange(off, off + nb[i])
            off += nb[i]
        ref = oracle.ref_decode(q.numpy().view(np.uint16), kp, vp, obt, lens, scale, "bf16")
        err = max_err(out.cpu().numpy(), ref)
        say(f"  decode rows={len(seqs)} plan={plan} max_err={err:.2e}")
        assert err <= ATOL
        return cplan


def test_system_prompt_hits_feed_decode(pkv):
    """64 users behind one 2,000-token system prompt: every later request matches the
    whole prompt (125 blocks) and writes only its own tokens; the prompt blocks stay
    bitwise as the first request wrote them; decode, plain and cascade, matches the
    oracle; the cascade plan finds the prompt as one node shared by all 64 rows."""
    say("radix: system prompt, 64 users")
    reqs = workloads.system_prompt_requests(seed=11, users=65, prompt_tokens=2000, user_lo=1, user_hi=300)
    h = Harness(pkv, 125 + 65 * 20 + 64, seed=1)
    assert h.admit(0, reqs[0]) == 0
    prompt_blocks = h.pool.table(0)[:125]
    k0 = h.k[torch.tensor(prompt_blocks).cuda()].clone()
    h.finish(0, reqs[0])
    for u in range(1, 65):
        assert h.admit(u, reqs[u]) == 2000
        assert h.pool.table(u)[:125] == prompt_blocks
    assert torch.equal(h.k[torch.tensor(prompt_blocks).cuda()], k0)
    seqs = list(range(1, 65))
    h.decode_and_check(seqs)
    plan = h.decode_and_check(seqs, plan=True)
    nodes = [plan.node(i) for i in range(plan.num_nodes)]
    assert any(len(b) >= 125 and len(m) == 64 for b, m in nodes), [(len(b), len(m)) for b, m in nodes]


@pytest.mark.parametrize("policy", ["lru", "rsbcm"])
def test_churn_with_eviction_keeps_live_requests_intact(pkv, policy):
    """A tight pool and a branching multi-turn request stream: finished requests are
    cached, new ones reuse prefixes, eviction frees unlocked leaves whose blocks are
    rewritten by later requests; the live (locked) requests still decode exactly
    as their logical records say."""
    say(f"radix: churn, policy={policy}")
    reqs = workloads.agent_sessions(seed=12, requests=160, prompts=3, prompt_lo=160, prompt_hi=600, msg_lo=8,
                                    msg_hi=64, open_max=8)
    h = Harness(pkv, 600, policy, seed=2)
    live = []
    for r, toks in enumerate(reqs):
        h.admit(r, toks)
        live.append(r)
        if len(live) > 8:
            done = live.pop(0)
            h.finish(done, reqs[done])
        if r % 40 == 39:
            h.decode_and_check(live)
    assert h.evictions > 0
    h.decode_and_check(live, plan=True)

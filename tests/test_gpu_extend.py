"""GPU parity: paged_extend_attn (multi-token causal attention on the matrix cores) against the
fp64 extend oracle, through the C ABI."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import ATOL, bits_np, device_setup, max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_21_amd as m

    return m


def run_extend(pkv, w, q, k_pages, v_pages, bt, lens, q_lens, min_members=2):
    torch = __import__("torch")
    plan = pkv.ExtendPlan(bt, lens, q_lens, w.num_q_heads, w.num_kv_heads, min_members=min_members).upload()
    out = pkv.paged_extend_attn(q, k_pages, v_pages, plan, scale=w.scale, dtype=w.dtype)
    torch.cuda.synchronize()
    return out.cpu().numpy(), plan


def make_q(w, rows, seed, device="cuda"):
    return workloads._normal_bits((rows, w.num_q_heads, w.head_dim), w.dtype, seed, device)


SHAPES = [
    ("bf16", 32, 8, 128),
    ("f16", 8, 8, 64),
    ("bf16", 16, 2, 128),
    ("f16", 64, 8, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}-hq{s[1]}-hkv{s[2]}-d{s[3]}" for s in SHAPES])
@pytest.mark.parametrize("seed", [0, 1])
def test_random_forest_extend_parity(pkv, shape, seed):
    """Forks at unaligned lengths, shared prefixes, ragged tails, rows without query tokens,
    a row whose every token is a query."""
    dtype, hq, hkv, d = shape
    w = workloads.random_forest(seed, num_rows=10, max_len=500, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, share_prob=0.6)
    pool, k_pages, v_pages = device_setup(w)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    rng = np.random.default_rng(100 + seed)
    q_lens = np.minimum(lens, rng.integers(0, 48, size=len(lens))).astype(np.int32)
    q_lens[0] = 0
    q_lens[1] = lens[1]  # every token of row 1 is a query (prefill from scratch)
    q = make_q(w, int(q_lens.sum()), 7 + seed)
    say(f"extend forest seed={seed} shape={shape} rows={int(q_lens.sum())}")
    ref = oracle.ref_extend(bits_np(q), bits_np(k_pages), bits_np(v_pages), bt, lens, q_lens, w.scale, dtype)
    for mm in (2, 1 << 20):  # with shared nodes, and every row on its own
        got, plan = run_extend(pkv, w, q, k_pages, v_pages, bt, lens, q_lens, min_members=mm)
        err = max_err(got, ref)
        say(f"  min_members={mm} nodes={plan.num_nodes} max_err={err:.3e}")
        assert err <= ATOL


@pytest.mark.parametrize("shape", [("bf16", 32, 8, 128), ("f16", 16, 16, 128)], ids=["bf16-gqa4", "f16-mha"])
def test_chunked_prefill_slice(pkv, shape):
    """A prompt slice of several hundred tokens over a long cached context: many 64-row tiles,
    many token pieces, pieces skipped for the early query tiles."""
    dtype, hq, hkv, d = shape
    w = workloads.random_forest(3, num_rows=2, max_len=2600, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, share_prob=0.0, min_len=2000)
    pool, k_pages, v_pages = device_setup(w)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    q_lens = np.asarray([333, 517], dtype=np.int32)
    q = make_q(w, int(q_lens.sum()), 21)
    got, plan = run_extend(pkv, w, q, k_pages, v_pages, bt, lens, q_lens)
    rows = sorted(set([0, 1, 63, 64, 200, 332, 333, 334, 600, 849]))
    ref = oracle.ref_extend(bits_np(q), bits_np(k_pages), bits_np(v_pages), bt, lens, q_lens, w.scale, dtype,
                            query_rows=rows)
    err = max_err(got[rows], ref)
    say(f"chunked prefill {shape}: max_err {err:.3e}")
    assert err <= ATOL and np.all(np.isfinite(got))


def test_verify_pass_over_shared_tree(pkv):
    """Branches of one search tree each score their last 8 tokens; the 256-token prefix is read
    once for all 32 query tokens per KV head."""
    w = workloads.get(1)
    pool, k_pages, v_pages = device_setup(w)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    q_lens = np.full(len(lens), 8, dtype=np.int32)
    q = make_q(w, int(q_lens.sum()), 5)
    got, plan = run_extend(pkv, w, q, k_pages, v_pages, bt, lens, q_lens)
    assert plan.num_nodes == 1 + len(lens)  # the shared prefix, and one private node per branch
    ref = oracle.ref_extend(bits_np(q), bits_np(k_pages), bits_np(v_pages), bt, lens, q_lens, w.scale, "f16")
    err = max_err(got, ref)
    say(f"verify tree: max_err {err:.3e}")
    assert err <= ATOL


def test_one_token_rows_match_decode(pkv):
    """q_lens = 1 everywhere is single-token decode: the extend pass and the split-K decode path
    agree within the tolerance."""
    w = workloads.random_forest(4, num_rows=9, max_len=900, dtype="bf16", num_q_heads=32, num_kv_heads=8,
                                head_dim=128, share_prob=0.5, min_len=1)
    pool, k_pages, v_pages = device_setup(w)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    q = make_q(w, len(lens), 9)
    got, _ = run_extend(pkv, w, q, k_pages, v_pages, bt, lens, np.ones(len(lens), dtype=np.int32))
    torch = __import__("torch")
    dec = pkv.paged_decode_attn(q, k_pages, v_pages, torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                                int(lens.max()), scale=w.scale, dtype="bf16")
    torch.cuda.synchronize()
    assert max_err(got, dec.cpu().numpy()) <= ATOL


def test_stale_nonfinite_rows_past_length(pkv):
    """Rows of a row's last block past its length hold Inf / NaN: masked, values zeroed."""
    w = workloads.random_forest(6, num_rows=6, max_len=400, dtype="f16", num_q_heads=8, num_kv_heads=8,
                                head_dim=64, share_prob=0.0, min_len=20)
    pool, k_pages, v_pages = device_setup(w)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    torch = __import__("torch")
    k_host, v_host = bits_np(k_pages).copy(), bits_np(v_pages).copy()
    for b in range(len(lens)):
        n = int(lens[b])
        if n % 16:
            blk = int(bt[b, n // 16])
            k_host[blk, n % 16:] = 0x7E00
            v_host[blk, n % 16:] = 0x7C00
    k_pages.copy_(torch.from_numpy(k_host.view(np.int16)).cuda())
    v_pages.copy_(torch.from_numpy(v_host.view(np.int16)).cuda())
    q_lens = np.minimum(lens, 19).astype(np.int32)
    q = make_q(w, int(q_lens.sum()), 3)
    got, _ = run_extend(pkv, w, q, k_pages, v_pages, bt, lens, q_lens)
    ref = oracle.ref_extend(bits_np(q), k_host, v_host, bt, lens, q_lens, w.scale, "f16")
    assert np.all(np.isfinite(got)) and max_err(got, ref) <= ATOL


def test_errors(pkv):
    torch = __import__("torch")
    w = workloads.get(1)
    pool, k_pages, v_pages = device_setup(w)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    with pytest.raises(pkv.PkvInvalid):
        pkv.ExtendPlan(bt, lens, lens + 1, w.num_q_heads, w.num_kv_heads)  # more queries than tokens
    dplan = pkv.CascadePlan(bt, lens, w.num_q_heads, w.num_kv_heads).upload()
    with pytest.raises(pkv.PkvInvalid):
        pkv.extend_workspace_bytes(dplan, w.head_dim)
    plan = pkv.ExtendPlan(bt, lens, np.full(len(lens), 2, np.int32), w.num_q_heads, w.num_kv_heads).upload()
    q = make_q(w, 2 * len(lens) + 1, 1)  # one row too many
    with pytest.raises(pkv.PkvInvalid):
        pkv.paged_extend_attn(q, k_pages, v_pages, plan, dtype="f16")

"""GPU parity for FP8 (E4M3) pages: the append kernel's codes and scales bit-exact against the
oracle's quantizer (copy-on-write included), and decode attention over FP8 pages against the fp64
oracle on the dequantized values, through the C ABI."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import ATOL, bits_np, max_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_21_amd as m

    return m


def to_dev(*arrays):
    torch = __import__("torch")
    return [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrays]


def quantized_pages(rng, nblk, bs, hkv, d, src_dtype):
    """Pages quantized by the oracle from N(0, 1) 16-bit values."""
    from oracle_checks import to_bits

    k16 = to_bits(rng.standard_normal((nblk, bs, hkv, d)), src_dtype)
    v16 = to_bits(rng.standard_normal((nblk, bs, hkv, d)), src_dtype)
    kc, ks = oracle.quantize_heads(oracle.decode_bits(k16, src_dtype))
    vc, vs = oracle.quantize_heads(oracle.decode_bits(v16, src_dtype))
    return kc, vc, np.ascontiguousarray(np.transpose(ks, (0, 2, 1))), np.ascontiguousarray(np.transpose(vs, (0, 2, 1)))


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("shape", [("bf16", 2, 64), ("f16", 8, 128)], ids=["bf16-hkv2-d64", "f16-hkv8-d128"])
def test_append_random_walk_bit_exact(pkv, seed, shape):
    torch = __import__("torch")
    dtype, hkv, d = shape
    rng = np.random.default_rng(900 + seed)
    nblk, bs = 40, 16
    order = rng.permutation(nblk)
    ref, lib = oracle.RefPool(nblk, bs, order), pkv.BlockPool(nblk, bs, order)
    kc, vc, ks, vs = quantized_pages(rng, nblk, bs, hkv, d, dtype)
    k_d, v_d, ks_d, vs_d = to_dev(kc, vc, ks.astype(np.float32), vs.astype(np.float32))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    next_seq, n_cow, n_tok = 0, 0, 0
    for it in range(100):
        live = ref.sequences()
        r = rng.random()
        if r < 0.12 or not live:
            n = int(rng.integers(0, 40))
            try:
                ref.alloc(next_seq, n)
            except MemoryError:
                continue
            lib.alloc(next_seq, n)
            next_seq += 1
        elif r < 0.4:
            parent = live[int(rng.integers(0, len(live)))]
            ref.fork(parent, next_seq)
            lib.fork(parent, next_seq)
            next_seq += 1
        elif r < 0.5:
            victim = live[int(rng.integers(0, len(live)))]
            ref.free(victim)
            lib.free(victim)
        else:
            k = int(rng.integers(1, len(live) + 1))
            batch = [live[i] for i in rng.permutation(len(live))[:k]]
            try:
                slots_r, cows_r = ref.plan_append(batch)
            except MemoryError:
                continue
            slots_l, cows_l = lib.plan_append(batch)
            assert list(slots_l) == slots_r
            n_cow += len(cows_r)
            n_tok += k
            # scaled so some vectors need large and some tiny scales; one all-zero head vector
            mult = torch.tensor(10.0 ** rng.integers(-6, 4, (k, 1, 1)), dtype=torch.float32, device="cuda")
            kn = (torch.randn((k, hkv, d), device="cuda") * mult).to(tdt)
            vn = (torch.randn((k, hkv, d), device="cuda") * mult).to(tdt)
            kn[0, 0] = 0
            cow = np.asarray(cows_l, dtype=np.int32).reshape(-1, 3)
            cow_d = to_dev(*(cow[:, i] for i in range(3))) if len(cow) else [None] * 3
            pkv.kv_append_fp8(k_d, v_d, ks_d, vs_d, kn, vn, torch.from_numpy(np.asarray(slots_l)).cuda(), *cow_d)
            kc, vc, ks, vs = oracle.apply_append_fp8(kc, vc, ks, vs, slots_r, cows_r, bits_np(kn.view(torch.int16)),
                                                     bits_np(vn.view(torch.int16)), dtype)
    torch.cuda.synchronize()
    say(f"fp8 append walk: {n_tok} tokens, {n_cow} copies")
    assert n_cow > 0
    assert np.array_equal(k_d.cpu().numpy(), kc) and np.array_equal(v_d.cpu().numpy(), vc)
    assert np.array_equal(ks_d.cpu().numpy(), ks) and np.array_equal(vs_d.cpu().numpy(), vs)


SHAPES = [("bf16", 32, 8, 128), ("f16", 8, 8, 64), ("bf16", 16, 2, 128), ("f16", 64, 8, 128)]


@pytest.mark.parametrize("use_plan", [False, True], ids=["split", "cascade"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}-hq{s[1]}-hkv{s[2]}-d{s[3]}" for s in SHAPES])
def test_decode_parity_random_forest(pkv, shape, use_plan):
    torch = __import__("torch")
    dtype, hq, hkv, d = shape
    w = workloads.random_forest(3, num_rows=12, max_len=900, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, share_prob=0.5)
    ref_pool = oracle.RefPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(ref_pool, w.build_ops, allow_cow=True)
    bt, lens = ref_pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    lens = lens.copy()
    lens[0] = 0
    rng = np.random.default_rng(77)
    kc, vc, ks, vs = quantized_pages(rng, w.num_blocks, w.block_size, hkv, d, dtype)
    # rows past every referencing row's length hold NaN codes and Inf scales: masked, never
    # read into the output
    valid = {}
    for b in range(len(lens)):
        n = int(lens[b])
        for j in range(-(-n // 16)):
            blk = int(bt[b, j])
            valid[blk] = max(valid.get(blk, 0), min(16, n - 16 * j))
    for blk in range(w.num_blocks):
        rows = valid.get(blk, 0)
        kc[blk, rows:] = 0x7F
        vc[blk, rows:] = 0x7F
        ks[blk, :, rows:] = np.inf
        vs[blk, :, rows:] = np.inf
    q = workloads._normal_bits((len(lens), hq, d), dtype, 13, "cuda")
    k_d, v_d, ks_d, vs_d, bt_d, l_d = to_dev(kc, vc, ks.astype(np.float32), vs.astype(np.float32), bt, lens)
    plan = None
    if use_plan:
        plan = pkv.CascadePlan(bt, lens, hq, hkv)
        assert plan.num_nodes > 0
        plan.upload(device="cuda")
    got = pkv.paged_decode_attn_fp8(q, k_d, v_d, ks_d, vs_d, bt_d, l_d, int(lens.max()), scale=w.scale, plan=plan,
                                    q_dtype=dtype)
    torch.cuda.synchronize()
    ref = oracle.ref_decode_fp8(bits_np(q), kc, vc, ks, vs, bt, lens, w.scale, dtype)
    err = max_err(got.cpu().numpy(), ref)
    say(f"fp8 decode {shape} plan={use_plan}: max_err {err:.3e}")
    assert np.all(np.isfinite(got.cpu().numpy())) and err <= ATOL
    assert np.all(got.cpu().numpy()[0] == 0)


def test_decode_llama8b_shape_sampled_rows(pkv):
    """The 8B-shaped layer with FP8 pages (codes and scales from the seeded generator)."""
    torch = __import__("torch")
    w = workloads.get(2)
    pool = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(pool, w.build_ops)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    kc, vc, ks, vs = workloads.make_fp8_pages(w, device="cuda")
    q = workloads.make_q(w, 0, device="cuda")
    bt_d, l_d = to_dev(bt, lens)
    got = pkv.paged_decode_attn_fp8(q, kc, vc, ks, vs, bt_d, l_d, int(lens.max()), scale=w.scale, q_dtype="bf16")
    torch.cuda.synchronize()
    rows = [0, 17, 40, 63]
    ids = sorted({int(x) for r in rows for x in bt[r, : -(-int(lens[r]) // 16)]})
    remap = {b: i for i, b in enumerate(ids)}
    idx = torch.tensor(ids, dtype=torch.int64, device="cuda")
    sub_bt = np.full((len(rows), bt.shape[1]), -1, np.int32)
    for i, r in enumerate(rows):
        nb = -(-int(lens[r]) // 16)
        sub_bt[i, :nb] = [remap[int(x)] for x in bt[r, :nb]]
    ref = oracle.ref_decode_fp8(bits_np(q)[rows], kc[idx].cpu().numpy(), vc[idx].cpu().numpy(),
                                ks[idx].cpu().numpy(), vs[idx].cpu().numpy(), sub_bt, lens[rows], w.scale, "bf16")
    err = max_err(got.cpu().numpy()[rows], ref)
    say(f"fp8 llama8b: max_err {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("cfg,rows", [(3, [0, 63, 64, 500, 1023]), (5, [0, 1, 100, 255])], ids=["tree-search", "radix"])
def test_tree_workloads_fp8_with_cascade_sampled_rows(pkv, cfg, rows):
    """The tree workloads at full size over FP8 pages, shared prefixes through the
    matrix-core pass: sampled rows against the oracle on the same codes and scales."""
    torch = __import__("torch")
    w = workloads.get(cfg)
    pool = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(pool, w.build_ops)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    kc, vc, ks, vs = workloads.make_fp8_pages(w, device="cuda")
    q = workloads.make_q(w, 0, device="cuda")
    bt_d, l_d = to_dev(bt, lens)
    plan = pkv.CascadePlan(bt, lens, w.num_q_heads, w.num_kv_heads)
    assert plan.num_nodes > 0
    plan.upload(device="cuda")
    got = pkv.paged_decode_attn_fp8(q, kc, vc, ks, vs, bt_d, l_d, int(lens.max()), scale=w.scale, plan=plan,
                                    q_dtype=w.dtype)
    plain = pkv.paged_decode_attn_fp8(q, kc, vc, ks, vs, bt_d, l_d, int(lens.max()), scale=w.scale, q_dtype=w.dtype)
    torch.cuda.synchronize()
    ids = sorted({int(x) for r in rows for x in bt[r, : -(-int(lens[r]) // 16)]})
    remap = {b: i for i, b in enumerate(ids)}
    idx = torch.tensor(ids, dtype=torch.int64, device="cuda")
    sub_bt = np.full((len(rows), bt.shape[1]), -1, np.int32)
    for i, r in enumerate(rows):
        nb = -(-int(lens[r]) // 16)
        sub_bt[i, :nb] = [remap[int(x)] for x in bt[r, :nb]]
    ref = oracle.ref_decode_fp8(bits_np(q)[rows], kc[idx].cpu().numpy(), vc[idx].cpu().numpy(),
                                ks[idx].cpu().numpy(), vs[idx].cpu().numpy(), sub_bt, lens[rows], w.scale, w.dtype)
    err = max_err(got.cpu().numpy()[rows], ref)
    err_plain = max_err(plain.cpu().numpy()[rows], ref)
    say(f"fp8 config {cfg} cascade: max_err {err:.3e} (split only {err_plain:.3e})")
    assert err <= ATOL and err_plain <= ATOL
    assert float((got - plain).abs().max()) <= 2 * ATOL


def test_errors(pkv):
    torch = __import__("torch")
    k = torch.zeros((4, 16, 2, 64), dtype=torch.uint8, device="cuda")
    s = torch.ones((4, 2, 16), dtype=torch.float32, device="cuda")
    q = torch.zeros((1, 2, 64), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    ln = torch.ones((1,), dtype=torch.int32, device="cuda")
    with pytest.raises((pkv.PkvUnsupported, ValueError)):
        pkv.paged_decode_attn_fp8(q.float(), k, k, s, s, bt, ln, 1)  # fp32 q
    lib = pkv.lib()
    assert lib.pkv_paged_decode_attn_fp8(q.data_ptr(), 1, 2, 2, 64, 1, k.data_ptr(), k.data_ptr(), None, None, 4, 16,
                                         bt.data_ptr(), 1, ln.data_ptr(), 1, 0.1, None, None, 0, None, None, None) == -1


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}-hq{s[1]}-hkv{s[2]}-d{s[3]}" for s in SHAPES])
def test_extend_parity_random_forest(pkv, shape):
    """Multi-token causal attention over FP8 pages (shared prefixes, ragged tails, a row
    without query tokens, a row whose every token is a query) against the FP8 extend oracle."""
    torch = __import__("torch")
    dtype, hq, hkv, d = shape
    w = workloads.random_forest(4, num_rows=10, max_len=500, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, share_prob=0.6)
    ref_pool = oracle.RefPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(ref_pool, w.build_ops, allow_cow=True)
    bt, lens = ref_pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    rng = np.random.default_rng(55)
    q_lens = np.minimum(lens, rng.integers(0, 40, size=len(lens))).astype(np.int32)
    q_lens[0] = 0
    q_lens[1] = lens[1]
    kc, vc, ks, vs = quantized_pages(rng, w.num_blocks, w.block_size, hkv, d, dtype)
    q = workloads._normal_bits((int(q_lens.sum()), hq, d), dtype, 21, "cuda")
    k_d, v_d, ks_d, vs_d = to_dev(kc, vc, ks.astype(np.float32), vs.astype(np.float32))
    plan = pkv.ExtendPlan(bt, lens, q_lens, hq, hkv).upload()
    got = pkv.paged_extend_attn_fp8(q, k_d, v_d, ks_d, vs_d, plan, scale=w.scale, q_dtype=dtype)
    torch.cuda.synchronize()
    ref = oracle.ref_extend_fp8(bits_np(q), kc, vc, ks, vs, bt, lens, q_lens, w.scale, dtype)
    err = max_err(got.cpu().numpy(), ref)
    say(f"fp8 extend {shape}: rows {int(q_lens.sum())} nodes {plan.num_nodes} max_err {err:.3e}")
    assert np.all(np.isfinite(got.cpu().numpy())) and err <= ATOL

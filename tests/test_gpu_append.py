"""GPU parity: kv_append (copy-on-write + slot scatter) bit-exact against the oracle, and the
radix-tree workload's append -> decode steps with backtracking against the oracle."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import ATOL, bits_np, max_err, say, tables_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_21_amd as m

    return m


def append_on_device(pkv, k_pages, v_pages, slots, cows, k_new, v_new, dtype):
    torch = __import__("torch")
    slot_d = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()
    if len(cows):
        c = np.ascontiguousarray(np.asarray(cows, dtype=np.int32).reshape(-1, 3))
        src, dst, rows = (torch.from_numpy(np.ascontiguousarray(c[:, i])).cuda() for i in range(3))
    else:
        src = dst = rows = None
    pkv.kv_append(k_pages, v_pages, k_new, v_new, slot_d, src, dst, rows, dtype=dtype)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("shape", [("bf16", 2, 64), ("f16", 8, 128)], ids=["bf16-hkv2-d64", "f16-hkv8-d128"])
def test_random_walk_pages_bit_exact(pkv, seed, shape):
    torch = __import__("torch")
    dtype, hkv, d = shape
    rng = np.random.default_rng(500 + seed)
    nblk, bs = 48, 16
    order = rng.permutation(nblk)
    ref = oracle.RefPool(nblk, bs, order)
    lib = pkv.BlockPool(nblk, bs, order)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    k_pages = torch.randn((nblk, bs, hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
    v_pages = torch.randn((nblk, bs, hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
    k_host, v_host = bits_np(k_pages), bits_np(v_pages)
    next_seq = 0
    n_cow = 0
    for it in range(120):
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
            kn = torch.randn((k, hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
            vn = torch.randn((k, hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
            append_on_device(pkv, k_pages, v_pages, slots_l, cows_l, kn, vn, dtype)
            k_host, v_host = oracle.apply_append(k_host, v_host, slots_r, cows_r, bits_np(kn), bits_np(vn))
    torch.cuda.synchronize()
    assert n_cow > 0
    assert np.array_equal(bits_np(k_pages), k_host)
    assert np.array_equal(bits_np(v_pages), v_host)


def test_padding_slots_are_skipped(pkv):
    torch = __import__("torch")
    k_pages = torch.zeros((4, 16, 2, 64), dtype=torch.int16, device="cuda")
    v_pages = torch.zeros_like(k_pages)
    kn = torch.full((3, 2, 64), 7, dtype=torch.int16, device="cuda")
    vn = torch.full((3, 2, 64), 9, dtype=torch.int16, device="cuda")
    slots = torch.tensor([5, -1, 63], dtype=torch.int64, device="cuda")
    pkv.kv_append(k_pages, v_pages, kn, vn, slots, dtype="bf16")
    k = k_pages.view(-1, 2, 64).cpu().numpy()
    v = v_pages.view(-1, 2, 64).cpu().numpy()
    assert np.all(k[5] == 7) and np.all(k[63] == 7) and np.all(v[63] == 9)
    assert int((k != 0).sum()) == 2 * 2 * 64


@pytest.mark.parametrize("fused", [False, True], ids=["two-calls", "one-launch"])
def test_radix_backtracking_protocol(pkv, fused):
    """Tree of 256 leaves over a 4096-token root; 16 steps of append -> decode with
    pruning / forking after steps 3, 7, 11, 15 (each fork shares a partly filled tail,
    so the next append copies it).  Pages bit-exact; every leaf compared at step 4 (the first
    after a backtrack, 64 copies on write) and step 16, sampled leaves at the other steps;
    either kv_append then paged_decode_attn, or paged_decode_attn_append."""
    torch = __import__("torch")
    w = workloads.get(5)
    k_pages, v_pages = workloads.make_pages(w, device="cuda")
    k_host, v_host = bits_np(k_pages), bits_np(v_pages)
    ref = oracle.RefPool(w.num_blocks, w.block_size, w.free_order)
    lib = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(ref, w.build_ops)
    workloads.replay(lib, w.build_ops)
    rng = np.random.default_rng(55)
    plan = None
    total_cow = 0
    for s, st in enumerate(w.steps):
        say(f"radix step {s + 1}")
        slots_r, cows_r = ref.plan_append(st.append_rows)
        slots_l, cows_l, row_src = lib.plan_append(st.append_rows, row_sources=True)
        assert list(slots_l) == slots_r
        assert [tuple(int(x) for x in c) for c in cows_l] == cows_r
        total_cow += len(cows_r)
        kn, vn = workloads.make_new_tokens(w, s, device="cuda")
        if not fused:
            append_on_device(pkv, k_pages, v_pages, slots_l, cows_l, kn, vn, "bf16")
        k_host, v_host = oracle.apply_append(k_host, v_host, slots_r, cows_r, bits_np(kn), bits_np(vn))
        bt, lens = lib.export_tables(st.decode_rows, w.max_blocks)
        bt_r, lens_r = ref.export_tables(st.decode_rows, w.max_blocks)
        assert np.array_equal(bt, bt_r) and np.array_equal(lens, lens_r)
        if plan is None:  # the tree changed (first step or after a backtrack): plan again
            plan = pkv.CascadePlan(bt, lens, w.num_q_heads, w.num_kv_heads).upload()
        bt_d, lens_d = tables_to_device(bt, lens)
        q = workloads.make_q(w, s, device="cuda")
        if fused:
            assert list(st.append_rows) == list(st.decode_rows)
            cow_src = torch.from_numpy(row_src).cuda()
            out = pkv.paged_decode_attn_append(q, k_pages, v_pages, bt_d, lens_d, int(lens.max()), kn, vn, cow_src,
                                               scale=w.scale, plan=plan, dtype="bf16")
        else:
            out = pkv.paged_decode_attn(q, k_pages, v_pages, bt_d, lens_d, int(lens.max()), scale=w.scale,
                                        plan=plan, dtype="bf16")
        if s in (3, 15):  # the first step after a backtrack (64 copies on write) and the last: every leaf
            assert s != 3 or len(cows_r) == 64
            rows = list(range(len(lens)))
        else:
            rows = sorted(rng.choice(len(lens), size=6, replace=False).tolist())
            # make sure a row that just copied a tail is among the checked ones
            if cows_r:
                touched = [i for i, sl in enumerate(slots_r) if sl // 16 == cows_r[0][1]]
                rows = sorted(set(rows + touched[:1]))
        got = out.cpu().numpy()[rows]
        refo = oracle.ref_decode_rows(bits_np(q), k_host, v_host, bt_r, lens_r, w.scale, "bf16", rows=rows)
        err = max_err(got, refo)
        say(f"  cows={len(cows_r)} rows={len(rows)} max_err={err:.3e}")
        assert err <= ATOL
        if s in (0, 3, 15):
            torch.cuda.synchronize()
            assert np.array_equal(bits_np(k_pages), k_host)
            assert np.array_equal(bits_np(v_pages), v_host)
        if st.after_ops:
            workloads.replay(ref, st.after_ops)
            workloads.replay(lib, st.after_ops)
            plan = None
    assert total_cow == 256

"""GPU parity of the one-launch append + decode (pkv_paged_decode_attn_append): pages
bit-exact against the oracle's apply_append, outputs within tolerance of the oracle's
decode over those pages, on random forests of forked sequences (shared partly filled
tails, so appends copy on write), with and without a cascade plan; plus the cases the
entry point must refuse or skip."""

import numpy as np
import pytest

import oracle
from gpu_util import ATOL, bits_np, max_err, say, tables_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_21_amd as m

    return m


def _forest(rng, ref, lib, roots, forks, max_len):
    """Roots of random lengths, then forks of random live sequences (children share
    every block, a partly filled tail included), then a few appends so that some
    shared tails are already copied."""
    seq = 0
    for _ in range(roots):
        n = int(rng.integers(1, max_len))
        ref.alloc(seq, n)
        lib.alloc(seq, n)
        seq += 1
    for _ in range(forks):
        live = ref.sequences()
        parent = live[int(rng.integers(0, len(live)))]
        ref.fork(parent, seq)
        lib.fork(parent, seq)
        seq += 1
    return seq


@pytest.mark.parametrize("plan_on", [False, True], ids=["split", "cascade"])
@pytest.mark.parametrize("shape", [("bf16", 32, 8, 128), ("f16", 8, 8, 64), ("bf16", 8, 2, 64), ("bf16", 32, 4, 128),
                                   ("f16", 16, 8, 128)],
                         ids=["bf16-g4-d128", "f16-g1-d64", "bf16-g4-d64", "bf16-g8-d128", "f16-g2-d128"])
@pytest.mark.parametrize("seed", range(2))
def test_fused_append_matches_oracle(pkv, seed, shape, plan_on):
    torch = __import__("torch")
    dtype, hq, hkv, d = shape
    say(f"fused append: seed={seed} shape={shape} plan={plan_on}")
    rng = np.random.default_rng(900 + seed)
    nblk, bs = 400, 16
    order = rng.permutation(nblk)
    ref = oracle.RefPool(nblk, bs, order)
    lib = pkv.BlockPool(nblk, bs, order)
    _forest(rng, ref, lib, roots=5, forks=23, max_len=700)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    k_pages = torch.randn((nblk, bs, hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
    v_pages = torch.randn((nblk, bs, hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
    k_host, v_host = bits_np(k_pages), bits_np(v_pages)
    total_cow = 0
    for step in range(3):
        live = ref.sequences()
        batch = [live[i] for i in rng.permutation(len(live))]
        slots_r, cows_r = ref.plan_append(batch)
        slots_l, cows_l, row_src = lib.plan_append(batch, row_sources=True)
        assert list(slots_l) == slots_r
        total_cow += len(cows_r)
        bt, lens = lib.export_tables(batch, 64)
        cow_src = row_src
        kn = torch.randn((len(batch), hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
        vn = torch.randn((len(batch), hkv, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
        q = torch.randn((len(batch), hq, d), generator=gen, device="cuda").to(tdt).view(torch.int16)
        plan = pkv.CascadePlan(bt, lens, hq, hkv).upload() if plan_on else None
        if plan_on:
            assert plan.num_nodes > 0
        bt_d, lens_d = tables_to_device(bt, lens)
        out = pkv.paged_decode_attn_append(q, k_pages, v_pages, bt_d, lens_d, int(lens.max()), kn, vn,
                                           torch.from_numpy(cow_src).cuda(), plan=plan, dtype=dtype)
        k_host, v_host = oracle.apply_append(k_host, v_host, slots_r, cows_r, bits_np(kn), bits_np(vn))
        torch.cuda.synchronize()
        assert np.array_equal(bits_np(k_pages), k_host), f"K pages differ at step {step}"
        assert np.array_equal(bits_np(v_pages), v_host), f"V pages differ at step {step}"
        refo = oracle.ref_decode(bits_np(q), k_host, v_host, bt, lens, 1.0 / np.sqrt(d), dtype)
        err = max_err(out.cpu().numpy(), refo)
        say(f"  step {step}: rows={len(batch)} cows={len(cows_r)} max_err={err:.3e}")
        assert err <= ATOL
    assert total_cow > 0


def test_fused_equals_append_then_decode(pkv):
    """Same inputs through kv_append + paged_decode_attn and through the fused call: the
    pages are bit-identical and the outputs agree to float rounding."""
    torch = __import__("torch")
    say("fused append vs two calls")
    rng = np.random.default_rng(77)
    nblk, bs, hq, hkv, d = 300, 16, 32, 8, 128
    order = rng.permutation(nblk)
    pools = [pkv.BlockPool(nblk, bs, order), pkv.BlockPool(nblk, bs, order)]
    refs = [oracle.RefPool(nblk, bs, order), oracle.RefPool(nblk, bs, order)]
    for ref, lib in zip(refs, pools):
        _forest(np.random.default_rng(5), ref, lib, roots=4, forks=20, max_len=900)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    k0 = torch.randn((nblk, bs, hkv, d), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    v0 = torch.randn((nblk, bs, hkv, d), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    ka, va, kb, vb = k0.clone(), v0.clone(), k0.clone(), v0.clone()
    batch = refs[0].sequences()
    slots, cows, row_src = pools[0].plan_append(batch, row_sources=True)
    slots_b, cows_b = pools[1].plan_append(batch)
    assert np.array_equal(slots, slots_b) and np.array_equal(cows, cows_b) and len(cows) > 0
    bt, lens = pools[0].export_tables(batch, 64)
    bt_d, lens_d = tables_to_device(bt, lens)
    kn = torch.randn((len(batch), hkv, d), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    vn = torch.randn((len(batch), hkv, d), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    q = torch.randn((len(batch), hq, d), generator=gen, device="cuda").to(torch.bfloat16).view(torch.int16)
    slot_d = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()
    c = np.ascontiguousarray(np.asarray(cows, dtype=np.int32).reshape(-1, 3))
    src, dst, rows = (torch.from_numpy(np.ascontiguousarray(c[:, i])).cuda() for i in range(3))
    pkv.kv_append(ka, va, kn, vn, slot_d, src, dst, rows, dtype="bf16")
    two = pkv.paged_decode_attn(q, ka, va, bt_d, lens_d, int(lens.max()), dtype="bf16")
    one = pkv.paged_decode_attn_append(q, kb, vb, bt_d, lens_d, int(lens.max()), kn, vn,
                                       torch.from_numpy(row_src).cuda(), dtype="bf16")
    torch.cuda.synchronize()
    assert torch.equal(ka, kb) and torch.equal(va, vb)
    assert float((one - two).abs().max()) <= 1e-5


def test_empty_rows_append_nothing_and_bad_plan_is_refused(pkv):
    torch = __import__("torch")
    say("fused append: empty rows, refused plan")
    nblk, bs, hkv, d = 8, 16, 2, 64
    k = torch.zeros((nblk, bs, hkv, d), dtype=torch.int16, device="cuda")
    v = torch.zeros_like(k)
    bt = np.array([[3, -1], [5, -1]], dtype=np.int32)
    lens = np.array([0, 1], dtype=np.int32)
    bt_d, lens_d = tables_to_device(bt, lens)
    kn = torch.full((2, hkv, d), 0x3F80, dtype=torch.int16, device="cuda")  # bf16 1.0
    vn = torch.full((2, hkv, d), 0x4000, dtype=torch.int16, device="cuda")  # bf16 2.0
    q = torch.zeros((2, hkv, d), dtype=torch.int16, device="cuda")
    cow = torch.tensor([-1, -1], dtype=torch.int32, device="cuda")
    out = pkv.paged_decode_attn_append(q, k, v, bt_d, lens_d, 1, kn, vn, cow, dtype="bf16")
    torch.cuda.synchronize()
    kk, vv = k.cpu().numpy(), v.cpu().numpy()
    assert np.all(kk[5, 0] == 0x3F80) and np.all(vv[5, 0] == 0x4000)
    assert int((kk != 0).sum()) == hkv * d and int((vv != 0).sum()) == hkv * d  # row 0 (length 0) wrote nothing
    o = out.cpu().numpy()
    assert np.all(o[0] == 0) and np.allclose(o[1], 2.0)
    # two rows whose last (full) block is shared: a plan from such tables is refused
    bt2 = np.array([[1, 2], [1, 2]], dtype=np.int32)
    lens2 = np.array([32, 32], dtype=np.int32)
    plan = pkv.CascadePlan(bt2, lens2, hkv, hkv).upload()
    bt2_d, lens2_d = tables_to_device(bt2, lens2)
    with pytest.raises(pkv.PkvInvalid):
        pkv.paged_decode_attn_append(q, k, v, bt2_d, lens2_d, 32, kn, vn, cow, plan=plan, dtype="bf16")
    torch.cuda.synchronize()


def test_clamped_rows_and_bad_cow_source(pkv):
    """A row longer than max_seq_len is attended up to max_seq_len and appends nothing; a
    copy-on-write source outside [0, num_blocks) is ignored (the row's own block is read
    and only the new token is written)."""
    torch = __import__("torch")
    say("fused append: clamped row, bad copy-on-write source")
    nblk, bs, hkv, d = 8, 16, 2, 64
    k = torch.zeros((nblk, bs, hkv, d), dtype=torch.int16, device="cuda")
    v = torch.zeros_like(k)
    v[2, :3] = 0x3F80  # row 1's own block: three tokens of V = 1.0 before the new one
    bt = np.array([[4, -1], [2, -1]], dtype=np.int32)
    lens = np.array([10, 4], dtype=np.int32)  # row 0 is longer than max_seq_len below
    bt_d, lens_d = tables_to_device(bt, lens)
    kn = torch.full((2, hkv, d), 0x3F80, dtype=torch.int16, device="cuda")
    vn = torch.full((2, hkv, d), 0x4040, dtype=torch.int16, device="cuda")  # bf16 3.0
    q = torch.zeros((2, hkv, d), dtype=torch.int16, device="cuda")
    cow = torch.tensor([-1, 99], dtype=torch.int32, device="cuda")
    out = pkv.paged_decode_attn_append(q, k, v, bt_d, lens_d, 6, kn, vn, cow, dtype="bf16")
    torch.cuda.synchronize()
    kk, vv = k.cpu().numpy(), v.cpu().numpy()
    assert not kk[4].any() and not vv[4].any()  # row 0 (clamped to 6 of its 10 tokens) wrote nothing
    assert np.all(vv[2, 3] == 0x4040) and np.all(kk[2, 3] == 0x3F80)  # row 1's token 3
    assert np.all(vv[2, :3] == 0x3F80) and not vv[2, 4:].any()
    o = out.cpu().numpy()
    assert np.allclose(o[0], 0.0)  # six zero tokens
    assert np.allclose(o[1], (1.0 + 1.0 + 1.0 + 3.0) / 4)  # uniform weights (q = 0)

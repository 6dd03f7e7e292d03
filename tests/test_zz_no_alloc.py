"""The decode entry point that allocates nothing (pkv_paged_decode_attn_noalloc):
called through the C ABI twice in a row on one device, the second time with a
smaller input, its output equals pkv_paged_decode_attn's with a caller workspace
(same kernels, same partial layout: bit for bit) and the oracle's within 2e-3;
sizes beyond the fixed scratch are refused on the host."""

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import ATOL, bits_np, device_setup, max_err, say, tables_to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pkv():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_21_amd as m

    return m


def _case(pkv, w, rows, cascade):
    torch = __import__("torch")
    pool, k_pages, v_pages = device_setup(w)
    bt, lens = pool.export_tables(rows, w.max_blocks)
    q = workloads.make_q(w, 0, device="cuda")[: len(rows)].contiguous()
    bt_d, lens_d = tables_to_device(bt, lens)
    plan = pkv.CascadePlan(bt, lens, w.num_q_heads, w.num_kv_heads).upload() if cascade else None
    if plan is not None and plan.num_nodes == 0:
        plan = None
    msl = int(max(lens.max(), 1))
    with_ws = pkv.paged_decode_attn(q, k_pages, v_pages, bt_d, lens_d, msl, scale=w.scale, plan=plan, dtype=w.dtype)
    out = torch.full_like(with_ws, float("nan"))
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.paged_decode_attn_noalloc(q, k_pages, v_pages, bt_d, lens_d, msl, out, scale=w.scale, plan=plan,
                                  dtype=w.dtype, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return with_ws, out, (q, k_pages, v_pages, bt, lens)


@pytest.mark.parametrize("cascade", [False, True], ids=["split", "cascade"])
def test_noalloc_matches_workspace_call_twice(pkv, cascade):
    torch = __import__("torch")
    # first call: the 8B-shaped layer (64 rows) or the radix tree (256 rows, shared nodes)
    w1 = workloads.get(5 if cascade else 2)
    rows1 = w1.steps[0].decode_rows
    say(f"noalloc call 1: workload {w1.number}, {len(rows1)} rows, cascade={cascade}")
    ref1, got1, _ = _case(pkv, w1, rows1, cascade)
    assert torch.equal(ref1, got1)
    # second call, smaller: a random forest of 9 rows (shared prefixes, ragged tails, empty rows)
    w2 = workloads.random_forest(3, num_rows=9, max_len=700, dtype="bf16", num_q_heads=32, num_kv_heads=8,
                                 head_dim=128, share_prob=0.6)
    rows2 = w2.steps[0].decode_rows
    say(f"noalloc call 2: random forest, {len(rows2)} rows, cascade={cascade}")
    ref2, got2, (q, k_pages, v_pages, bt, lens) = _case(pkv, w2, rows2, cascade)
    assert torch.equal(ref2, got2)
    expect = oracle.ref_decode(bits_np(q), bits_np(k_pages), bits_np(v_pages), bt, lens, w2.scale, w2.dtype)
    assert max_err(got2.cpu().numpy(), expect) <= ATOL


def test_noalloc_refuses_sizes_beyond_the_scratch(pkv):
    torch = __import__("torch")
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    pages = torch.zeros((4, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((64, 4096), dtype=torch.int32, device="cuda")
    lens = torch.ones((64,), dtype=torch.int32, device="cuda")
    out = torch.empty((64, 32, 128), dtype=torch.float32, device="cuda")
    need = pkv.decode_workspace_bytes(64, 32, 8, 128, 65536)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pkv.PkvWorkspaceError):
        pkv.paged_decode_attn_noalloc(q, pages, pages, bt, lens, 65536, out)

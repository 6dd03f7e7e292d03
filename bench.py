"""Throughput of one paged decode step on one MI355X.

A step is the whole hot path over one batch: append one new token per sequence
(kv_append, slots planned on the host by the library's block pool), then
single-token decode attention over every sequence's paged KV cache
(paged_decode_attn: cascade pass over shared blocks when a plan has any,
split-K partial attention over each row's own blocks, partial merge).  Host
planning (append plan, cascade plan) is timed separately and reported.

Default workload: the Llama-3-8B-shaped decode layer (64 sequences, lengths
uniform in [512, 4096], Hq=32, Hkv=8, d=128, bf16 K/V, 16-token blocks,
random placement).  ``--config 1..5`` selects the other synthetic workloads.

Prints one JSON line.  ``value`` = effective unique-KV GB/s of the step: the
distinct K/V bytes the step must read plus q, output and table bytes, divided
by the measured step time (inputs resident in HBM, back-to-back steps).

``--extend`` measures the multi-token pass instead (paged_extend_attn): the
verify pass over the tree-search workload (``--config 3``: the last 8 tokens
of every branch) or a chunked-prefill slice (``--config 6``: 4,096 tokens over
28,672 cached), reported as causal attention TFLOP/s against the matrix-core
peak.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}  # MI355X dense matrix-core peak per dtype


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first: a few hundred bring the GPU to its steady clocks (with 10 the "
                         "8B step timed 4-7 %% slower)")
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5, 6],
                    help="time this workload alone (default: the 8B-shaped layer as the headline, then a line "
                         "per other workload)")
    ap.add_argument("--fp8", action="store_true",
                    help="FP8 (E4M3) pages with per-row scales: quantizing append + FP8 decode (configs 2 and 4)")
    ap.add_argument("--protocol", action="store_true",
                    help="run every step of a multi-step workload (the radix tree's 16 append + decode steps "
                         "with backtracking), timing host planning and device work per step")
    ap.add_argument("--swap", action="store_true",
                    help="block swap between HBM and pinned host memory: GB/s each way, overlap with decode")
    ap.add_argument("--swap-blocks", type=int, default=16384, help="blocks per swap batch (32 KiB of K and of V each)")
    ap.add_argument("--radix", action="store_true",
                    help="host prefix cache: request throughput and hit rate on request traces (no GPU work)")
    ap.add_argument("--extend", action="store_true",
                    help="time the multi-token pass (configs 3: verify 8 tokens per branch, 6: chunked prefill)")
    ap.add_argument("--no-cascade", action="store_true", help="decode every row on its own (no shared-prefix pass)")
    ap.add_argument("--fused", action="store_true",
                    help="step = the one-launch paged_decode_attn_append (default: kv_append then paged_decode_attn)")
    ap.add_argument("--cold-iters", type=int, default=50,
                    help="decode calls (and steps) each preceded by a 1 GiB write that evicts L2 and MALL (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the oracle baseline (0 = skip)")
    ap.add_argument("--read-ceiling-gib", type=int, default=4,
                    help="also time a plain streaming read of this many GiB (the read-bandwidth yardstick; 0 = skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (for scaling HBM counters)")
    return ap.parse_args()


def read_ceiling(gib, dev):
    """Best median GB/s of the library's plain streaming read over `gib` GiB, over a few grid sizes."""
    import torch

    import paged_kv_cache_21_amd as pkv

    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = (0.0, 0)
    for grid in (1024, 2048, 4096, 8192):
        times = []
        for it in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            pkv.stream_read(buf, sink, grid)
            e1.record()
            torch.cuda.synchronize()
            if it:
                times.append(e0.elapsed_time(e1))
        gbs = buf.numel() / (float(np.median(times)) * 1e-3) / 1e9
        best = max(best, (gbs, grid))
    # freed into torch's cache, not back to the driver: device memory mapped again after a
    # release measured 2-4 % slower under the same kernels (FP8 8B split 63.7 -> 66.1 us),
    # so no workload of this run is timed on memory the driver has just handed back
    del buf
    return {"gbs": round(best[0], 1), "grid": best[1], "bytes": gib << 30,
            "kernel": "stream_read_kernel (16-byte non-temporal loads, 4 in flight per thread)"}


def unique_bytes(bt, lens, w):
    """Distinct K/V bytes one decode reads: valid tokens of every distinct block referenced."""
    per_block = {}
    for b in range(len(lens)):
        n = int(lens[b])
        nb = -(-n // w.block_size)
        for j in range(nb):
            valid = min(w.block_size, n - j * w.block_size)
            blk = int(bt[b, j])
            per_block[blk] = max(per_block.get(blk, 0), valid)
    return sum(per_block.values()) * w.bytes_per_token


def host_rows(q_bits, k_pages, v_pages, bt, lens, rows):
    """Host copies of the inputs the given decode rows read (their blocks, renumbered)."""
    import torch

    bs = k_pages.shape[1]
    ids = []
    for r in rows:
        ids.extend(int(x) for x in bt[r, : -(-int(lens[r]) // bs)])
    uniq = sorted(set(ids)) or [0]
    remap = {b: i for i, b in enumerate(uniq)}
    idx = torch.tensor(uniq, dtype=torch.int64, device=k_pages.device)
    k = k_pages.index_select(0, idx).cpu().numpy().view(np.uint16)
    v = v_pages.index_select(0, idx).cpu().numpy().view(np.uint16)
    sbt = np.full((len(rows), bt.shape[1]), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        nb = -(-int(lens[r]) // bs)
        sbt[i, :nb] = [remap[int(x)] for x in bt[r, :nb]]
    qb = q_bits[list(rows)].cpu().numpy().view(np.uint16) if q_bits is not None else None
    return k, v, sbt, np.asarray([lens[r] for r in rows], dtype=np.int32), qb


def host_cores():
    """The host's CPU count and this process's affinity, reported beside the oracle baseline
    (which runs on one thread with one BLAS thread)."""
    return {"host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "blas_threads": 1}


def cpu_baseline(w, q_bits, k_pages, v_pages, bt, lens, seconds):
    """Time the fp64 oracle (one BLAS thread) over the workload's rows, row after row
    and pass after pass, until about `seconds` of oracle time has been spent."""
    import oracle
    from threadpoolctl import threadpool_limits

    rows_done = 0
    tokens = 0
    t_total = 0.0
    passes = 0
    with threadpool_limits(limits=1):
        while t_total < seconds:
            for b in range(len(lens)):
                k, v, sbt, sl, qb = host_rows(q_bits, k_pages, v_pages, bt, lens, [b])
                t0 = time.perf_counter()
                oracle.ref_decode(qb, k, v, sbt, sl, w.scale, w.dtype)
                t_total += time.perf_counter() - t0
                rows_done += 1
                tokens += int(lens[b])
                if t_total >= seconds:
                    break
            passes += 1
    gbs = tokens * w.bytes_per_token / t_total / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle", **host_cores(),
            "sample": f"{rows_done} decode rows ({passes} pass(es) over the {len(lens)} rows of the workload, "
                      f"{tokens} tokens, all {w.num_q_heads} query heads), {t_total:.1f} s of fp64 numpy oracle "
                      f"time on one host thread; {rows_done / t_total:.2f} decode queries/s"}


def measured_traffic(w, kernel_source="paged_kv_cache_21_amd/csrc/decode.hip"):
    """HBM bytes per split-kernel launch from the committed PMC summary, if it was taken on this
    workload with this exact kernel source (else None)."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))["decode_split_kernel"]
    except (OSError, KeyError, ValueError):
        return None
    src = os.path.join(ROOT, kernel_source)
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != digest or rec.get("workload") != w.name:
        return None
    kib = rec["fetch_kib_per_dispatch"] * rec["fetch_scale"] + rec["write_kib_per_dispatch"] * rec["write_scale"]
    return int(round(kib * 1024))


def extend_cpu_baseline(w, q_bits, k_pages, v_pages, bt, lens, q_lens, seconds):
    """Time the fp64 extend oracle (one BLAS thread) over a sample of query rows spread over the
    workload, until about `seconds` of oracle time; returns causal flop/s."""
    import oracle
    from threadpoolctl import threadpool_limits

    where = oracle.extend_query_positions(lens, q_lens)
    rng = np.random.default_rng(0)
    order = rng.permutation(len(where))
    done, flops, t_total = 0, 0.0, 0.0
    rows = {}
    with threadpool_limits(limits=1):
        for r in order:
            b, pos = where[int(r)]
            if b not in rows:
                rows = {b: host_rows(None, k_pages, v_pages, bt, lens, [b])}
            k, v, sbt, sl, _ = rows[b]
            qrow = q_bits[int(r):int(r) + 1].cpu().numpy().view(np.uint16)
            t0 = time.perf_counter()
            # the row cut after the query's position, with the query as its one new token
            oracle.ref_extend(qrow, k, v, sbt, np.asarray([pos + 1], np.int32), np.asarray([1], np.int32), w.scale,
                              w.dtype)
            t_total += time.perf_counter() - t0
            done += 1
            flops += 4.0 * w.head_dim * (pos + 1) * w.num_q_heads
            if t_total >= seconds:
                break
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle", **host_cores(),
            "sample": f"{done} query rows drawn at random from the workload's {len(where)} (all {w.num_q_heads} "
                      f"heads each), {t_total:.1f} s of fp64 numpy oracle time on one host thread"}


def run_extend(args, w, dev, emit=True):
    """Multi-token pass: one paged_extend_attn call per step over the workload's query tokens."""
    import torch

    import paged_kv_cache_21_amd as pkv
    import workloads

    if args.fp8:
        k_pages, v_pages, k_scales, v_scales = workloads.make_fp8_pages(w, device=dev)
    else:
        k_pages, v_pages = workloads.make_pages(w, device=dev)
    pool = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(pool, w.build_ops)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    q_lens = np.minimum(lens, workloads.EXTEND_QUERY_TOKENS[w.number]).astype(np.int32)
    t0 = time.perf_counter()
    plan = pkv.ExtendPlan(bt, lens, q_lens, w.num_q_heads, w.num_kv_heads)
    plan_us = (time.perf_counter() - t0) * 1e6
    plan.upload(device=dev)
    nq = int(q_lens.sum())
    q = workloads._normal_bits((nq, w.num_q_heads, w.head_dim), w.dtype, 1000 + w.seed, dev)
    ws = torch.empty(pkv.extend_workspace_bytes(plan, w.head_dim), dtype=torch.uint8, device=dev)
    out = torch.empty((nq, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def one_step():
        if args.fp8:
            pkv.paged_extend_attn_fp8(q, k_pages, v_pages, k_scales, v_scales, plan, scale=w.scale, workspace=ws,
                                      out=out, q_dtype=w.dtype, stream=stream)
        else:
            pkv.paged_extend_attn(q, k_pages, v_pages, plan, scale=w.scale, workspace=ws, out=out, dtype=w.dtype,
                                  stream=stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        one_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / max(args.steps, 1)
    pkv.timing_reset()
    pkv.timing_enable(True)
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    pkv.timing_enable(False)
    kern = {}
    for name in ("cascade", "merge"):
        total, count = pkv.timing_read(name)
        kern[name] = {"avg_us": round(total / count * 1e3, 3) if count else 0.0, "launches": count}

    # causal flops: 2*d per (query, head, attended token) for q.k and again for p.v
    first = lens - q_lens
    attended = int(sum(int(q_lens[b]) * int(first[b]) + int(q_lens[b]) * (int(q_lens[b]) + 1) // 2
                       for b in range(len(lens))))
    flops = 4.0 * w.head_dim * w.num_q_heads * attended
    kv_unique = unique_bytes(bt, lens, w)
    t_mfma = kern["cascade"]["avg_us"] * 1e-6
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    achieved = flops / t_mfma / 1e12 if t_mfma > 0 else 0.0
    cpu = None
    if args.cpu_seconds > 0 and not args.fp8:
        cpu = extend_cpu_baseline(w, q, k_pages, v_pages, bt, lens, q_lens, args.cpu_seconds)
    res = {
        "metric": "paged extend attn: causal attention TFLOP/s, effective unique-KV GB/s",
        "value": round(flops / (ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 pages, " + w.dtype + " q" if args.fp8 else w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}" + ("; FP8 pages" if args.fp8 else ""), "query_tokens": nq, "rows": int((q_lens > 0).sum()),
                   "query_tokens_per_row": int(workloads.EXTEND_QUERY_TOKENS[w.number]),
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "shared_nodes": plan.num_nodes, "accumulate": "f32",
                   "parallelism": "single GPU"},
        "effective_kv_gbs": round(kv_unique / (ms * 1e-3) / 1e9, 1),
        "hbm_peak_frac": round(kv_unique / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "attended_token_pairs": attended,
        "kernels": kern,
        "host_us": {"plan_build": round(plan_us, 1)},
        "roofline": {"bound": "mfma", "kernel": "cascade_kernel", "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "algorithmic_flops_per_launch": flops, "avg_launch_us": kern["cascade"]["avg_us"]},
        "cpu_baseline": cpu,
    }
    if emit:
        print(json.dumps(res), flush=True)
    return res


def run_fp8(args, w, dev, emit=True):
    """Append + decode over FP8 pages (with the shared-prefix pass when the workload shares
    blocks): the decode's K/V bytes halve."""
    import torch

    import paged_kv_cache_21_amd as pkv
    import workloads

    kc, vc, ks, vs = workloads.make_fp8_pages(w, device=dev)
    pool = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(pool, w.build_ops)
    slots, cows = pool.plan_append(w.steps[0].append_rows)
    cow = np.asarray(cows, dtype=np.int32).reshape(-1, 3)
    cow_d = [torch.from_numpy(np.ascontiguousarray(cow[:, i])).to(dev) for i in range(3)] if len(cow) else [None] * 3
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    plan = None if args.no_cascade else pkv.CascadePlan(bt, lens, w.num_q_heads, w.num_kv_heads)
    if plan is not None and plan.num_nodes == 0:
        plan = None
    if plan is not None:
        plan.upload(device=dev)
    q = workloads.make_q(w, 0, device=dev)
    k_new, v_new = workloads.make_new_tokens(w, 0, device=dev)
    slot_d, bt_d, lens_d = (torch.from_numpy(x).to(dev) for x in (slots, bt, lens))
    max_len = int(lens.max())
    B = len(lens)
    ws = torch.empty(max(pkv.decode_workspace_bytes(B, w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, plan), 16),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((B, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def one_step():
        pkv.kv_append_fp8(kc, vc, ks, vs, k_new, v_new, slot_d, cow_d[0], cow_d[1], cow_d[2], src_dtype=w.dtype,
                          stream=stream)
        pkv.paged_decode_attn_fp8(q, kc, vc, ks, vs, bt_d, lens_d, max_len, scale=w.scale, plan=plan, workspace=ws,
                                  out=out, q_dtype=w.dtype, stream=stream)

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        one_step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / max(args.steps, 1)
    pkv.timing_reset()
    pkv.timing_enable(True)
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    pkv.timing_enable(False)
    kern = {}
    for name in ("append", "decode_split", "merge", "cascade"):
        total, count = pkv.timing_read(name)
        kern[name] = {"avg_us": round(total / count * 1e3, 3) if count else 0.0, "launches": count}
    # bytes per token of one layer: codes (1 B per element, K and V) + one fp32 scale per head for K and V
    per_token = w.num_kv_heads * (2 * w.head_dim + 2 * 4)
    tokens = int(lens.sum())
    unique_tokens = unique_bytes(bt, lens, w) // w.bytes_per_token  # distinct cached tokens referenced
    own_tokens = sum(int(lens[b]) - plan.row(b)[0] for b in range(B)) if plan is not None else tokens
    q_bytes = B * w.num_q_heads * w.head_dim * 2
    split_bytes = own_tokens * per_token + q_bytes
    U = unique_tokens * per_token + q_bytes + B * w.num_q_heads * w.head_dim * 4 + bt.nbytes + lens.nbytes
    t_split = kern["decode_split"]["avg_us"] * 1e-6
    achieved = split_bytes / t_split / 1e9 if t_split > 0 else 0.0
    res = {
        "metric": "paged decode attn over FP8 pages: effective KV GB/s, decode queries/s",
        "value": round(U / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}; K/V as E4M3 codes with per-row fp32 power-of-two scales",
                   "batch": B, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "q_dtype": w.dtype, "accumulate": "f32", "cascade": plan is not None,
                   "parallelism": "single GPU"},
        "decode_queries_per_s": round(B / (ms * 1e-3), 1),
        "tokens_per_s_equivalent_16bit_gbs": round(tokens * w.bytes_per_token / (ms * 1e-3) / 1e9, 1),
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel<FP8>", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": split_bytes, "avg_launch_us": kern["decode_split"]["avg_us"]},
        "cpu_baseline": None,
    }
    if emit:
        print(json.dumps(res), flush=True)
    return res


def radix_replay(Pool, Cache, reqs, num_blocks, policy, block_size=16, batch=32, seconds=None, meta=None):
    """Serve ``reqs`` in order through a prefix cache, ``batch`` at a time: one batched
    admission (each request matches all but its last token, locks it, evicts when
    the pool is short, starts on the matched blocks), then one batched completion
    (cache the full blocks with their (score, depth) from ``meta``, unlock,
    release).  Requests that did not fit go first
    in the next batch.  Returns (requests done, seconds, matched tokens, total
    tokens, admission calls)."""
    pool = Pool(num_blocks, block_size)
    cache = Cache(pool, policy)
    hits = total = done = calls = 0
    queue = list(range(len(reqs)))
    t0 = time.perf_counter()
    while queue:
        ids = queue[:batch]
        got = cache.admit([reqs[i] for i in ids], ids)
        calls += 1
        if not got:
            raise RuntimeError(f"request {ids[0]} does not fit in a pool of {num_blocks} blocks")
        adm = ids[:len(got)]
        cache.finish([reqs[i] for i in adm], adm, [n for _, n in got],
                     None if meta is None else [meta[i][0] for i in adm],
                     None if meta is None else [meta[i][1] for i in adm])
        queue = ids[len(got):] + queue[batch:]
        for (m, _), i in zip(got, adm):
            hits += m
            total += len(reqs[i])
        done += len(got)
        if seconds is not None and time.perf_counter() - t0 > seconds:
            break
    return done, time.perf_counter() - t0, hits, total, calls


def run_radix(args):
    """Host prefix cache on two request traces: the RadixAttention section's 1,000
    users behind one 2,000-token system prompt, and a multi-turn, branching agent
    stream over 8 system prompts in a pool of 4,096 blocks, far fewer than its
    distinct blocks (so leaves are evicted), under both eviction orders.  Requests
    go through batched admission and completion, 32 per call.  The library is
    timed; the oracle serves a bounded prefix of the same traces the same way."""
    import oracle
    import paged_kv_cache_21_amd as pkv
    import workloads

    agent, agent_meta = workloads.agent_sessions(seed=8, requests=4000, meta=True)
    traces = [
        ("system_prompt_1000x2000", workloads.system_prompt_requests(seed=7), None, 1 << 16, "lru"),
        ("agent_sessions_4000_lru", agent, agent_meta, 4096, "lru"),
        ("agent_sessions_4000_rsbcm", agent, agent_meta, 4096, "rsbcm"),
    ]
    per = {}
    total_req = total_s = 0.0
    for name, reqs, meta, nblk, policy in traces:
        radix_replay(pkv.BlockPool, pkv.RadixCache, reqs[:50], nblk, policy, meta=meta)  # warm-up
        done, sec, hits, tok, calls = radix_replay(pkv.BlockPool, pkv.RadixCache, reqs, nblk, policy, meta=meta)
        per[name] = {"requests": done, "us_per_request": round(sec / done * 1e6, 2),
                     "hit_rate": round(hits / tok, 4), "admission_calls": calls, "pool_blocks": nblk,
                     "tokens_per_request": round(tok / done, 1)}
        total_req += done
        total_s += sec
        print(f"[bench] radix {name}: {done} requests, {sec / done * 1e6:.1f} us/request, "
              f"hit rate {hits / tok:.3f}, {calls} admission calls", file=sys.stderr, flush=True)
    value = total_req / total_s
    cpu = None
    if args.cpu_seconds > 0:
        c_req = c_s = 0.0
        for name, reqs, meta, nblk, policy in traces:
            done, sec, _, _, _ = radix_replay(oracle.RefPool, oracle.RadixCache, reqs, nblk, policy,
                                              seconds=args.cpu_seconds / len(traces), meta=meta)
            c_req += done
            c_s += sec
        cpu = {"value": round(c_req / c_s, 2), "unit": "requests/s", "cores": 1, "kind": "oracle", **host_cores(),
               "sample": f"first {int(c_req)} requests over the three traces, about {args.cpu_seconds:.0f} s"}
    line = {"metric": "prefix_cache_requests_per_s", "value": round(value, 1), "unit": "requests/s",
            "n_gpus": 0, "steps": int(total_req), "warmup": 150, "ms_per_step": round(total_s / total_req * 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
            "data": "synthetic", "config": {"workload": "prefix cache request traces", "traces": per},
            "roofline": None, "cpu_baseline": cpu}
    print(json.dumps(line))


def run_protocol(args, w, dev):
    """All steps of a multi-step workload as a serving loop would run them: per step the
    host plans the append (slots, copy-on-write list) and exports the tables, replans
    the shared-prefix pass when the tree changed (after a backtrack), then the device
    appends and decodes.  Device time per step from events around its kernels; host
    time per step from the host clock; effective GB/s over each step's unique bytes."""
    import torch

    import paged_kv_cache_21_amd as pkv
    import workloads

    k_pages, v_pages = workloads.make_pages(w, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run_once(record):
        pool = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
        workloads.replay(pool, w.build_ops)
        plan = None
        ws = None
        for s, st in enumerate(w.steps):
            t0 = time.perf_counter()
            slots, cows = pool.plan_append(st.append_rows)
            t1 = time.perf_counter()
            bt, lens = pool.export_tables(st.decode_rows, w.max_blocks)
            replanned = plan is None
            if replanned:
                plan = pkv.CascadePlan(bt, lens, w.num_q_heads, w.num_kv_heads)
            t2 = time.perf_counter()
            max_len = int(lens.max())
            need = pkv.decode_workspace_bytes(len(lens), w.num_q_heads, w.num_kv_heads, w.head_dim, max_len, plan)
            if ws is None or ws.numel() < need:
                ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
            if replanned:
                plan.upload(device=dev)
            kn, vn = workloads.make_new_tokens(w, s, device=dev)
            q = workloads.make_q(w, s, device=dev)
            slot_d = torch.from_numpy(slots).to(dev)
            cow = np.asarray(cows, dtype=np.int32).reshape(-1, 3)
            cow_d = ([torch.from_numpy(np.ascontiguousarray(cow[:, i])).to(dev) for i in range(3)] if len(cow)
                     else [None] * 3)
            bt_d, lens_d = torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev)
            out = torch.empty((len(lens), w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pkv.kv_append(k_pages, v_pages, kn, vn, slot_d, cow_d[0], cow_d[1], cow_d[2], dtype=w.dtype,
                          stream=stream)
            pkv.paged_decode_attn(q, k_pages, v_pages, bt_d, lens_d, max_len, scale=w.scale, plan=plan,
                                  workspace=ws, out=out, dtype=w.dtype, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            if record is not None:
                U = (unique_bytes(bt, lens, w) + len(lens) * w.num_q_heads * w.head_dim * 6 + bt.nbytes +
                     lens.nbytes)
                record.append({"step": s + 1, "device_us": round(e0.elapsed_time(e1) * 1e3, 2),
                               "plan_append_us": round((t1 - t0) * 1e6, 1),
                               "export_and_plan_us": round((t2 - t1) * 1e6, 1), "replanned": replanned,
                               "copy_on_write": len(cow), "gb_per_s": round(U / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)})
            if st.after_ops:
                workloads.replay(pool, st.after_ops)
                plan = None

    run_once(None)  # warm-up pass
    steps = []
    run_once(steps)
    dev_us = [x["device_us"] for x in steps]
    host_us = [x["plan_append_us"] + x["export_and_plan_us"] for x in steps]
    line = {"metric": "multi-step decode protocol: device time per step, effective KV GB/s", "value":
            round(float(np.mean([x["gb_per_s"] for x in steps])), 1), "unit": "GB/s", "n_gpus": 1,
            "steps": len(steps), "warmup": len(steps), "ms_per_step": round(float(np.mean(dev_us)) / 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
            "config": {"workload": f"{w.name}: {w.description}", "per_step": steps},
            "host_us_per_step_mean": round(float(np.mean(host_us)), 1),
            "copy_on_write_total": int(sum(x["copy_on_write"] for x in steps)),
            "roofline": None, "cpu_baseline": None}
    print(json.dumps(line), flush=True)


def run_swap(args, dev):
    """Swap traffic of the 8B-shaped layer (Hkv 8, d 128, bf16: 32 KiB of K and 32 KiB
    of V per block): ``--swap-blocks`` scattered blocks out to scattered pinned host
    slots and back, one pkv_copy_blocks launch per direction (K and V together).
    Beside it: the same copies as runtime copies (per block, and in runs of 16
    blocks), the rate of one contiguous copy of the same size (hipMemcpyAsync
    through torch), and 40 decode steps of the 8B workload run alone, back to back
    with a swap-in of a quarter of the blocks, and concurrently with it on a second
    stream."""
    import torch

    import paged_kv_cache_21_amd as pkv
    import workloads

    n = int(args.swap_blocks)
    hkv, d = 8, 128
    per_block = 2 * 16 * hkv * d * 2
    rng = np.random.default_rng(21)
    k = torch.randint(-2 ** 15, 2 ** 15 - 1, (n, 16, hkv, d), dtype=torch.int16, device=dev)
    v = torch.randint(-2 ** 15, 2 ** 15 - 1, (n, 16, hkv, d), dtype=torch.int16, device=dev)
    hk = torch.empty((n, 16, hkv, d), dtype=torch.int16, pin_memory=True)
    hv = torch.empty((n, 16, hkv, d), dtype=torch.int16, pin_memory=True)
    dev_ids = torch.from_numpy(rng.permutation(n).astype(np.int32)).to(dev)
    host_ids = torch.from_numpy(rng.permutation(n).astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    reps = max(args.steps // 10, 3)
    out_ms = timed(lambda: pkv.copy_blocks([hk, hv], [k, v], host_ids, dev_ids, stream=stream), reps)
    in_ms = timed(lambda: pkv.copy_blocks([k, v], [hk, hv], dev_ids, host_ids, stream=stream), reps)
    dev_np, host_np = dev_ids.cpu().numpy(), host_ids.cpu().numpy()
    mc_out_ms = timed(lambda: pkv.copy_blocks_memcpy([hk, hv], [k, v], host_np, dev_np, stream=stream), reps)
    mc_in_ms = timed(lambda: pkv.copy_blocks_memcpy([k, v], [hk, hv], dev_np, host_np, stream=stream), reps)
    # runs of 16 consecutive blocks on both sides (256-token pieces of sequences), in shuffled order
    run = 16
    perm_d, perm_h = rng.permutation(n // run), rng.permutation(n // run)
    run_dev = (perm_d[:, None] * run + np.arange(run)[None, :]).reshape(-1).astype(np.int32)
    run_host = (perm_h[:, None] * run + np.arange(run)[None, :]).reshape(-1).astype(np.int32)
    mc_run_in_ms = timed(lambda: pkv.copy_blocks_memcpy([k, v], [hk, hv], run_dev, run_host, stream=stream), reps)
    capped = {}
    for g in (16, 32, 64, 128, 256):
        capped[g] = timed(lambda: pkv.copy_blocks([k, v], [hk, hv], dev_ids, host_ids, stream=stream,
                                                  max_workgroups=g), reps)
    # the last swap-out and swap-in moved the same bytes: sampled blocks agree
    chk = torch.from_numpy(rng.integers(0, n, size=64)).to(dev)
    assert torch.equal(k[dev_ids[chk].long()].cpu(), hk[host_ids[chk].long().cpu()])
    # the link's own rate: one contiguous copy of the same bytes each way
    kf, hkf = k.view(-1), hk.view(-1)
    d2h_ms = timed(lambda: hkf.copy_(kf, non_blocking=True), reps) * 2   # K only: scale to K+V
    h2d_ms = timed(lambda: kf.copy_(hkf, non_blocking=True), reps) * 2
    gb = n * per_block / 1e9
    out_gbs, in_gbs, d2h_gbs, h2d_gbs = gb / (out_ms / 1e3), gb / (in_ms / 1e3), gb / (d2h_ms / 1e3), gb / (h2d_ms / 1e3)
    mc_out_gbs, mc_in_gbs = gb / (mc_out_ms / 1e3), gb / (mc_in_ms / 1e3)
    mc_run_in_gbs = gb / (mc_run_in_ms / 1e3)
    print(f"[bench] swap {n} blocks ({gb:.2f} GB): kernel out {out_ms:.2f} ms = {out_gbs:.1f} GB/s, "
          f"in {in_ms:.2f} ms = {in_gbs:.1f} GB/s; runtime copies per block out {mc_out_gbs:.1f}, "
          f"in {mc_in_gbs:.1f} GB/s, in runs of {run} {mc_run_in_gbs:.1f} GB/s; "
          f"contiguous copy d2h {d2h_gbs:.1f}, h2d {h2d_gbs:.1f} GB/s", file=sys.stderr, flush=True)

    # overlap: decode steps of the 8B workload with a concurrent swap-in of a quarter of the blocks
    w = workloads.get(2)
    kp, vp = workloads.make_pages(w, device=dev)
    pool = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(pool, w.build_ops)
    bt, lens = pool.export_tables(w.steps[0].decode_rows, w.max_blocks)
    q = workloads.make_q(w, 0, device=dev)
    bt_d, lens_d = torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev)
    max_len = int(lens.max())
    ws = torch.empty(pkv.decode_workspace_bytes(len(lens), w.num_q_heads, w.num_kv_heads, w.head_dim, max_len),
                     dtype=torch.uint8, device=dev)
    o = torch.empty((len(lens), w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    side = torch.cuda.Stream(dev)
    m = n // 4
    sub_dev, sub_host = dev_ids[:m].contiguous(), host_ids[:m].contiguous()
    sub_dev_np, sub_host_np = run_dev[:m].copy(), run_host[:m].copy()
    steps = 40

    def decode_steps(st):
        for _ in range(steps):
            pkv.paged_decode_attn(q, kp, vp, bt_d, lens_d, max_len, scale=w.scale, workspace=ws, out=o,
                                  dtype=w.dtype, stream=st)

    cap = [0]

    def swap_in(st):
        if cap[0] < 0:
            pkv.copy_blocks_memcpy([k, v], [hk, hv], sub_dev_np, sub_host_np, stream=st)
        else:
            pkv.copy_blocks([k, v], [hk, hv], sub_dev, sub_host, stream=st, max_workgroups=cap[0])

    def wall(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3

    def both():
        side.wait_stream(stream)
        swap_in(side)
        decode_steps(stream)
        stream.wait_stream(side)

    t_dec = wall(lambda: decode_steps(stream))
    overlap = {}
    for g in (0, 32, -1):
        cap[0] = g
        t_swp = wall(lambda: swap_in(stream))
        t_serial = wall(lambda: (decode_steps(stream), swap_in(stream)))
        t_both = wall(both)
        hidden = (t_serial - t_both) / min(t_dec, t_swp) if min(t_dec, t_swp) > 0 else 0.0
        overlap[g] = {"swap_in_ms": round(t_swp, 3), "back_to_back_ms": round(t_serial, 3),
                      "concurrent_ms": round(t_both, 3), "hidden_fraction": round(hidden, 3)}
        how = "runtime copies, runs of 16" if g < 0 else f"copy kernel, {g or 'one work-group per block'}"
        print(f"[bench] overlap ({how}): {steps} decode steps {t_dec:.2f} ms, "
              f"swap-in of {m} blocks {t_swp:.2f} ms, back to back {t_serial:.2f} ms, concurrent {t_both:.2f} ms "
              f"({hidden:.0%} of the shorter hidden)", file=sys.stderr, flush=True)
    line = {"metric": "swap_in_gb_per_s", "value": round(in_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": reps,
            "warmup": 2, "ms_per_step": round(in_ms, 4), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"swap of {n} scattered blocks, Hkv 8, d 128, bf16 (K and V, {per_block} B per block)",
                       "swap_out_gb_per_s": round(out_gbs, 2), "contiguous_copy_d2h_gb_per_s": round(d2h_gbs, 2),
                       "contiguous_copy_h2d_gb_per_s": round(h2d_gbs, 2),
                       "swap_in_gb_per_s_by_workgroups": {str(g): round(gb / (t / 1e3), 2) for g, t in capped.items()},
                       "overlap": {"decode_steps": steps, "decode_ms": round(t_dec, 3), "swap_in_blocks": m,
                                   "by_path": {("runtime_copies" if g < 0 else f"kernel_{g}"): v for g, v in overlap.items()}},
                       "runtime_copies_per_block_out_gb_per_s": round(mc_out_gbs, 2),
                       "runtime_copies_per_block_in_gb_per_s": round(mc_in_gbs, 2),
                       "runtime_copies_runs_of_16_in_gb_per_s": round(mc_run_in_gbs, 2)},
            "roofline": {"bound": "host link", "achieved": round(in_gbs, 2), "peak": 64.0, "unit": "GB/s",
                         "frac": round(in_gbs / 64.0, 4), "traffic": None,
                         "frac_of_contiguous_copy": round(in_gbs / h2d_gbs, 4)},
            "cpu_baseline": None}
    print(json.dumps(line))


# The decode step timed for each workload: the first step, except for the radix tree,
# where it is the first step after a backtrack (its append copies 64 shared tails on write).
TIMED_STEP = {1: 0, 2: 0, 3: 0, 4: 0, 5: 3}
HEADLINE_CONFIG = 2
EXTRA_CONFIGS = (1, 3, 4, 5)


def setup_step(w, dev, step_index, cascade):
    """Pages, the library pool replayed to the timed step, that step's append plan and
    tables, and the cascade plan (None when off or when nothing is shared)."""
    import types

    import torch

    import paged_kv_cache_21_amd as pkv
    import workloads

    r = types.SimpleNamespace()
    r.k_pages, r.v_pages = workloads.make_pages(w, device=dev)
    pool = pkv.BlockPool(w.num_blocks, w.block_size, w.free_order)
    workloads.replay(pool, w.build_ops)
    for s_ in range(step_index):  # earlier steps on the host pool only (values do not matter for timing)
        pool.plan_append(w.steps[s_].append_rows)
        if w.steps[s_].after_ops:
            workloads.replay(pool, w.steps[s_].after_ops)
    step = w.steps[step_index]
    t0 = time.perf_counter()
    r.slots, r.cows, r.row_src = pool.plan_append(step.append_rows, row_sources=True)
    r.plan_append_us = (time.perf_counter() - t0) * 1e6
    r.fused_ok = list(step.append_rows) == list(step.decode_rows)
    r.bt, r.lens = pool.export_tables(step.decode_rows, w.max_blocks)
    t0 = time.perf_counter()
    plan = pkv.CascadePlan(r.bt, r.lens, w.num_q_heads, w.num_kv_heads) if cascade else None
    r.plan_build_us = (time.perf_counter() - t0) * 1e6
    if plan is not None and plan.num_nodes == 0:
        plan = None
    if plan is not None:
        plan.upload(device=dev)
    r.plan = plan
    r.q = workloads.make_q(w, step_index, device=dev)
    r.k_new, r.v_new = workloads.make_new_tokens(w, step_index, device=dev)
    r.slot_d = torch.from_numpy(r.slots).to(dev)
    cow = np.asarray(r.cows, dtype=np.int32).reshape(-1, 3)
    r.cow_d = ([torch.from_numpy(np.ascontiguousarray(cow[:, i])).to(dev) for i in range(3)] if len(cow)
               else [None] * 3)
    r.cow_src_d = torch.from_numpy(r.row_src).to(dev)
    r.bt_d = torch.from_numpy(r.bt).to(dev)
    r.lens_d = torch.from_numpy(r.lens).to(dev)
    r.max_len = int(r.lens.max())
    need = max(pkv.decode_workspace_bytes(len(r.lens), w.num_q_heads, w.num_kv_heads, w.head_dim, r.max_len, plan),
               pkv.decode_workspace_bytes(len(r.lens), w.num_q_heads, w.num_kv_heads, w.head_dim, r.max_len))
    r.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    r.out = torch.empty((len(r.lens), w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    r.stream = torch.cuda.current_stream(dev)
    B = len(r.lens)
    r.kv_unique = unique_bytes(r.bt, r.lens, w)
    r.kv_logical = int(r.lens.sum()) * w.bytes_per_token
    r.q_bytes = B * w.num_q_heads * w.head_dim * 2
    r.o_bytes = B * w.num_q_heads * w.head_dim * 4
    r.tbl_bytes = r.bt.nbytes + r.lens.nbytes
    r.U = r.kv_unique + r.q_bytes + r.o_bytes + r.tbl_bytes
    return r


def step_fns(w, r, fused, use_plan=True):
    """(one step = append + decode, the decode call alone) for the set-up r."""
    import paged_kv_cache_21_amd as pkv

    plan = r.plan if use_plan else None

    def attn_call():
        pkv.paged_decode_attn(r.q, r.k_pages, r.v_pages, r.bt_d, r.lens_d, r.max_len, scale=w.scale, plan=plan,
                              workspace=r.ws, out=r.out, dtype=w.dtype, stream=r.stream)

    def one_step():
        if fused:  # append + decode in one launch
            pkv.paged_decode_attn_append(r.q, r.k_pages, r.v_pages, r.bt_d, r.lens_d, r.max_len, r.k_new, r.v_new,
                                         r.cow_src_d, scale=w.scale, plan=plan, workspace=r.ws, out=r.out,
                                         dtype=w.dtype, stream=r.stream)
            return
        pkv.kv_append(r.k_pages, r.v_pages, r.k_new, r.v_new, r.slot_d, r.cow_d[0], r.cow_d[1], r.cow_d[2],
                      dtype=w.dtype, stream=r.stream)
        attn_call()

    return one_step, attn_call


def time_back_to_back(fn, stream, steps, warmup):
    """ms per call over `steps` back-to-back calls after `warmup` untimed ones (inputs resident)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / max(steps, 1)


def time_flushed(fn, stream, iters, dev, flush=None):
    """Per-call ms, each call preceded by a 1 GiB write that evicts L2 and the 256 MB MALL
    (the first call untimed): list of `iters` times."""
    import torch

    own = flush is None
    if own:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    out = []
    for it in range(iters + 1):
        flush.fill_(it & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        if it:
            out.append(e0.elapsed_time(e1))
    if own:
        del flush
    return out


def pct(xs):
    """(median, p10, p90) of a list of ms, in us."""
    a = np.asarray(xs) * 1e3
    return round(float(np.median(a)), 3), round(float(np.percentile(a, 10)), 3), round(float(np.percentile(a, 90)), 3)


def kernel_times(fn, steps):
    """Per-kernel average us from the library's event timing over `steps` calls."""
    import torch

    import paged_kv_cache_21_amd as pkv

    pkv.timing_reset()
    pkv.timing_enable(True)
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    pkv.timing_enable(False)
    kern = {}
    for name in ("append", "decode_split", "merge", "cascade"):
        total, count = pkv.timing_read(name)
        kern[name] = {"avg_us": round(total / count * 1e3, 3) if count else 0.0, "launches": count}
    return kern


def summarize_config(w, dev, steps, warmup, flush_iters, flush):
    """One workload's line in the default run: warm step and decode-call times, the flushed
    decode call (median, p10, p90), per-kernel times, bytes, with and without the cascade
    pass when the workload shares blocks."""
    import torch

    r = setup_step(w, dev, TIMED_STEP[w.number], cascade=True)
    one_step, attn_call = step_fns(w, r, fused=False)
    step_ms = time_back_to_back(one_step, r.stream, steps, warmup)
    attn_ms = time_back_to_back(attn_call, r.stream, steps, warmup)
    fl = pct(time_flushed(attn_call, r.stream, flush_iters, dev, flush))
    kern = kernel_times(one_step, steps)
    out = {"workload": f"{w.name}: {w.description}", "timed_step": TIMED_STEP[w.number] + 1, "rows": len(r.lens),
           "copy_on_write": len(r.cows), "step_us": round(step_ms * 1e3, 3), "decode_call_us": round(attn_ms * 1e3, 3),
           "decode_call_flushed_us_median_p10_p90": list(fl),
           "effective_gb_per_s": round(r.U / (attn_ms * 1e-3) / 1e9, 1),
           "effective_gb_per_s_flushed_median": round(r.U / (fl[0] * 1e-6) / 1e9, 1),
           "hbm_peak_frac": round(r.U / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "decode_queries_per_s": round(len(r.lens) / (attn_ms * 1e-3), 1),
           "bytes": {"unique_U": r.U, "kv_unique": r.kv_unique, "kv_logical": r.kv_logical},
           "kernels_us": {k: v["avg_us"] for k, v in kern.items() if v["launches"]},
           "cascade": r.plan is not None, "shared_nodes": r.plan.num_nodes if r.plan is not None else 0,
           "host_us": {"plan_append": round(r.plan_append_us, 1), "plan_build": round(r.plan_build_us, 1)}}
    if r.fused_ok:  # the same step as one launch (pkv_paged_decode_attn_append)
        fused_step, _ = step_fns(w, r, fused=True)
        out["step_us_one_launch"] = round(time_back_to_back(fused_step, r.stream, steps, warmup) * 1e3, 3)
    if r.plan is not None:  # the same call with every row decoded on its own
        _, attn_off = step_fns(w, r, fused=False, use_plan=False)
        off_ms = time_back_to_back(attn_off, r.stream, steps, warmup)
        off_fl = pct(time_flushed(attn_off, r.stream, flush_iters, dev, flush))
        kern_off = kernel_times(attn_off, steps)
        out["cascade_off"] = {"decode_call_us": round(off_ms * 1e3, 3),
                              "decode_call_flushed_us_median_p10_p90": list(off_fl),
                              "kernels_us": {k: v["avg_us"] for k, v in kern_off.items() if v["launches"]},
                              "speedup_of_cascade": round(off_ms / attn_ms, 3)}
    del r  # (kept in torch's cache: see read_ceiling)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by rows / heads with no exchange, but nothing here launches more than one GPU).",
              file=sys.stderr)
        sys.exit(2)

    if args.radix:
        return run_radix(args)

    import torch

    import paged_kv_cache_21_amd as pkv
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.swap:
        return run_swap(args, dev)
    default_run = args.config is None
    w = workloads.get(HEADLINE_CONFIG if default_run else args.config)
    print(f"[bench] workload {w.number} {w.name}: {w.description}", file=sys.stderr, flush=True)
    if args.protocol:
        return run_protocol(args, w, dev)
    if args.extend or w.number == 6:
        return run_extend(args, w, dev)
    if args.fp8:
        return run_fp8(args, w, dev)

    # ---- set-up (not timed): pages, pool, the step's append plan, tables, cascade plan
    r = setup_step(w, dev, TIMED_STEP[w.number], cascade=not args.no_cascade)
    fused = args.fused
    if fused and not r.fused_ok:
        print("--fused needs the step to append one token to every decoded row", file=sys.stderr)
        sys.exit(2)
    one_step, attn_call = step_fns(w, r, fused)
    plan, lens, bt, cows = r.plan, r.lens, r.bt, r.cows

    # ---- timed region 1: K back-to-back steps (the reported value)
    ms_per_step = time_back_to_back(one_step, r.stream, args.steps, args.warmup)

    # ---- timed region 2: the same K steps with per-kernel HIP events (library timing, same stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pkv.timing_reset()
    pkv.timing_enable(True)
    torch.cuda.synchronize()
    ev0.record(r.stream)
    for _ in range(args.steps):
        one_step()
    ev1.record(r.stream)
    torch.cuda.synchronize()
    pkv.timing_enable(False)
    ms_per_step_instrumented = ev0.elapsed_time(ev1) / max(args.steps, 1)
    kern = {}
    for name in ("append", "decode_split", "merge", "cascade"):
        total, count = pkv.timing_read(name)
        kern[name] = {"avg_us": round(total / count * 1e3, 3) if count else 0.0, "launches": count}

    # ---- flushed: each call after a 1 GiB write that evicts L2 and the 256 MB MALL
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.cold_iters > 0 else None
    cold = time_flushed(one_step, r.stream, args.cold_iters, dev, flush) if args.cold_iters > 0 else []
    attn_cold = time_flushed(attn_call, r.stream, args.cold_iters, dev, flush) if args.cold_iters > 0 else []

    if args.copy_calibration_mib > 0:
        src = torch.empty(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(3)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.copy_calibration_mib} MiB read + written", file=sys.stderr)

    # ---- bytes
    B = len(lens)
    U = r.U
    value = U / (ms_per_step * 1e-3) / 1e9

    # roofline of the dominant kernel: split-K decode; algorithmic bytes = the K/V of every row's own
    # (not shared) tokens plus q, per launch
    if plan is not None:
        own_tokens = sum(int(lens[b]) - plan.row(b)[0] for b in range(B))
    else:
        own_tokens = int(lens.sum())
    split_bytes = own_tokens * w.bytes_per_token + r.q_bytes
    if fused:  # the split kernel also reads the new tokens and writes them and the copied-on-write rows
        split_bytes += (2 * B + sum(int(c[2]) for c in cows)) * w.bytes_per_token
    t_split = kern["decode_split"]["avg_us"] * 1e-6
    achieved = split_bytes / t_split / 1e9 if t_split > 0 else 0.0
    traffic = measured_traffic(w) if plan is None or plan.num_nodes == 0 else None
    roofline = {"bound": "hbm", "kernel": "decode_split_kernel", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "traffic_unit": "bytes per launch (HBM read + write, rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
                "algorithmic_bytes_per_launch": split_bytes, "avg_launch_us": kern["decode_split"]["avg_us"]}

    # the paged_decode_attn call alone (no append): K back-to-back calls on the same inputs
    t_attn = time_back_to_back(attn_call, r.stream, args.steps, args.warmup) * 1e-3
    attn_gbs = U / t_attn / 1e9 if t_attn > 0 else 0.0
    attn_only = {"us": round(t_attn * 1e6, 3), "gb_per_s": round(attn_gbs, 1),
                 "hbm_peak_frac": round(attn_gbs / HBM_PEAK_GBS, 4)}
    flushed = None
    if attn_cold:
        med, p10, p90 = pct(attn_cold)
        flushed = {"decode_call_us_median": med, "decode_call_us_p10": p10, "decode_call_us_p90": p90,
                   "gb_per_s_median": round(U / (med * 1e-6) / 1e9, 1),
                   "hbm_peak_frac_median": round(U / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                   "decode_queries_per_s_median": round(B / (med * 1e-6), 1), "iterations": len(attn_cold)}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, r.q, r.k_pages, r.v_pages, bt, lens, args.cpu_seconds)
    ceiling = read_ceiling(args.read_ceiling_gib, dev) if args.read_ceiling_gib > 0 else None
    if ceiling:
        roofline["frac_of_measured_read_ceiling"] = round(achieved / ceiling["gbs"], 4)

    res = {
        "metric": "paged decode attn: effective KV GB/s, % of HBM peak, decode queries/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": B, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "mean_seq_len": round(float(lens.mean()), 1), "max_seq_len": r.max_len, "accumulate": "f32",
                   "cascade": plan is not None, "shared_nodes": plan.num_nodes if plan is not None else 0,
                   "step": "paged_decode_attn_append (one launch)" if fused else "kv_append + paged_decode_attn",
                   "parallelism": "single GPU"},
        "headline": "value = unique bytes U / ms_per_step, warm back-to-back steps (kv_append + paged_decode_attn) "
                    "with inputs resident in HBM; decode_attn_only = the decode call alone, warm; flushed = the "
                    "decode call after a 1 GiB write each time (median, p10, p90)",
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_queries_per_s": round(B / (ms_per_step * 1e-3), 1),
        "decode_attn_only": attn_only,
        "flushed": flushed,
        "bytes": {"kv_unique": r.kv_unique, "kv_logical": r.kv_logical, "q": r.q_bytes, "out": r.o_bytes,
                  "tables": r.tbl_bytes, "step_total_U": U},
        "kernels": kern,
        "ms_per_step_instrumented": round(ms_per_step_instrumented, 5),
        "cold_ms_per_step_median": round(float(np.median(cold)), 5) if cold else None,
        "cold_ms_per_step_p10_p90": [round(float(np.percentile(cold, 10)), 5),
                                     round(float(np.percentile(cold, 90)), 5)] if cold else None,
        "host_us": {"plan_append": round(r.plan_append_us, 1), "plan_build": round(r.plan_build_us, 1)},
        "roofline": roofline,
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
    }
    if default_run and not args.no_cascade and not fused:
        del r  # (kept in torch's cache: see read_ceiling)
        configs = {}
        for n in EXTRA_CONFIGS:
            wx = workloads.get(n)
            print(f"[bench] workload {n} {wx.name}", file=sys.stderr, flush=True)
            configs[f"config{n}"] = summarize_config(wx, dev, steps=max(args.steps // 2, 10), warmup=args.warmup,
                                                    flush_iters=max(args.cold_iters, 10), flush=flush)
        res["configs"] = configs
        # the FP8 and multi-token passes, timed in the same run (shorter timed loops, the full
        # warm-up so the clocks are steady, no oracle)
        import argparse as _ap
        sub = _ap.Namespace(**vars(args))
        sub.steps, sub.warmup, sub.cpu_seconds = max(args.steps // 5, 10), args.warmup, 0.0
        extras = {}
        for key, n, kind in (("fp8_decode_8b", 2, "fp8"), ("fp8_decode_70b_mha", 4, "fp8"),
                             ("extend_tree_verify", 3, "extend"), ("extend_chunked_prefill", 6, "extend")):
            wx = workloads.get(n)
            print(f"[bench] {key}: workload {n} {wx.name}", file=sys.stderr, flush=True)
            sub.fp8 = kind == "fp8"
            rx = run_fp8(sub, wx, dev, emit=False) if kind == "fp8" else run_extend(sub, wx, dev, emit=False)
            extras[key] = {k: rx[k] for k in ("value", "unit", "ms_per_step", "dtype", "kernels", "roofline")}
            extras[key]["workload"] = rx["config"]["workload"]
        res["extras"] = extras
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Decode-step benchmark of the paged-KV attention path on one MI355X.

Headline step (the 7B-shaped batch): 64 sequences with context lengths
uniform in [128, 4096], 32 query heads = 32 kv heads, head_dim 128,
block_size 16, blocks shuffled across a 200,000-block pool, bf16 K/V, fp32
accumulation.  One step appends one token to every sequence: pa_cache_write
of the new K/V rows into the slots the host allocator assigned, then
pa_decode (partition kernel + split-K reduce) over the grown contexts.
Inputs are synthetic (seeded N(0,1)) and resident in HBM: the allocator runs
ahead of the timed region for every step, and its slots, block tables and
lengths are uploaded before timing starts.  The allocator's own host cost and
the rate with per-step host work and PCIe uploads in the loop are reported
beside `value`, never as it.

Prints one JSON line.  `value` = decoded tokens per second.  `roofline`
covers pa_decode, timed with HIP events on its launch stream inside the
timed region.  `rows` measures the other steps of the path on their own
workloads (grouped-query decode, prefix-shared decode with copy-on-write,
long-context split-K decode, chunked prefill, the mixed step, cache write,
block copy, allocator).  `cpu_baseline` is the fp64 oracle on the same batch.

Counter runs: `--calibrate` adds one plain block copy of known size (1 GiB
read + 1 GiB written) after the timed loop; `--pmc-summary FETCH_DIR
WRITE_DIR` turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) into
the per-launch HBM traffic file the `traffic` field reads.
"""
from __future__ import annotations

import argparse
import csv
import gc
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode tokens/s and achieved KV HBM GB/s (% of MI355X peak), 1 GPU"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mha_7b_traffic.json")
# the decode partition kernel: the longest-first scan grid (batches of up to
# 256 sequences, as every bench workload) or the slot grid
DECODE_KERNEL = ("decode_scan_kernel", "decode_mfma_kernel")
KERNEL_SOURCES = ("decode_mfma.hip", "decode_reduce.hip", "decode_split.h", "device_common.h", "launch.h")
CALIB_PAIRS = 4096
HOST_WARM = 4  # untimed steps before the host-inclusive loop's timed ones


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_417_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def decode_bytes(lengths, hq, hkv, d, bs, e_kv=2, e_q=2):
    """Algorithmic bytes of one decode call: K and V of every valid token,
    q, the fp32 output, the block-table entries read and the lengths."""
    kv = sum(int(L) for L in lengths) * hkv * d * 2 * e_kv
    s = len(lengths)
    tables = sum(-(-int(L) // bs) for L in lengths) * 4
    return kv + s * hq * d * e_q + s * hq * d * 4 + tables + s * 4


def prefill_flops(ctx, qlens, hq, d):
    """QK^T and PV flops of causal chunks: row i of a chunk sees ctx-qlen+i+1 keys."""
    total = 0
    for c, q in zip(ctx, qlens):
        c, q = int(c), int(q)
        keys = q * (c - q) + q * (q + 1) // 2
        total += 4 * hq * d * keys
    return total


def measured_traffic(src_hash: str):
    """HBM bytes per decode launch from the committed counter runs, if they
    were taken on this exact kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def events_time(torch, fn, reps, stream):
    """Per-call milliseconds of fn() from HIP events on `stream`."""
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ts)
    return ms[len(ms) // 2], ms


def spread(ms) -> dict:
    """p10 / p90 of a row's per-call times (sorted milliseconds), in us."""
    return {"p10_us": ms[len(ms) // 10] * 1e3, "p90_us": ms[(9 * len(ms)) // 10] * 1e3}


def warm(torch, fn, seconds: float) -> None:
    """Untimed calls of fn() for about `seconds`: the matrix-bound prefill
    runs well below its steady rate until the chip's clocks have ramped
    under it (after the memory-bound rows its first calls are ~20% slower)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# CPU baseline


def _oracle_helpers():
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paged_helpers import gather_blocks, host_bits
    return oracle, gather_blocks, host_bits


def oracle_decode_sample(case, budget_s: float, tables=None, lengths=None, scales=(1.0, 1.0)):
    """The fp64 oracle, single-threaded, on whole sequences of a decode batch
    (all heads) until the time budget is spent or the batch is done.
    Returns (sequences done, context tokens, seconds)."""
    oracle, gather_blocks, host_bits = _oracle_helpers()
    sh = case.shape
    tabs = case.tables if tables is None else tables
    lens = case.lengths if lengths is None else lengths
    done, elapsed, tokens = 0, 0.0, 0
    for s in range(len(lens)):
        k_sub, v_sub, t_sub, l_sub = gather_blocks(case.k_pool, case.v_pool, tabs, lens, [s],
                                                   sh.block_size)
        q_sub = host_bits(case.q[s:s + 1])
        t0 = time.perf_counter()
        oracle.decode(q_sub, k_sub, v_sub, t_sub, l_sub, sh.scale, case.k_axes, case.v_axes,
                      scales[0], scales[1])
        elapsed += time.perf_counter() - t0
        done += 1
        tokens += int(l_sub[0])
        if elapsed >= budget_s:
            break
    return done, tokens, elapsed


def host_threads() -> int:
    """Worker threads for the all-core oracle run: the cores this process may
    use, at most 16 (one GPU's share of the host: the box gives a one-GPU job
    16 CPUs whatever nproc shows; `host_cpus` in the result is nproc)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_decode_parallel(case, budget_s: float, threads: int):
    """The same fp64 oracle over the whole decode batch, one sequence per
    task on ``threads`` host threads (the C oracle runs outside the GIL).
    Each sequence's blocks are copied to the host once, untimed; the batch
    is repeated until the budget is spent.  Returns (batches, tokens, s)."""
    from concurrent.futures import ThreadPoolExecutor
    oracle, gather_blocks, host_bits = _oracle_helpers()
    sh = case.shape
    lens = case.lengths
    work = []
    for s in range(len(lens)):
        k_sub, v_sub, t_sub, l_sub = gather_blocks(case.k_pool, case.v_pool, case.tables, lens,
                                                   [s], sh.block_size)
        work.append((host_bits(case.q[s:s + 1]), k_sub, v_sub, t_sub, l_sub))

    def one(w):
        oracle.decode(w[0], w[1], w[2], w[3], w[4], sh.scale, case.k_axes, case.v_axes)

    one(work[0])  # loads the oracle library before the threads start
    reps, elapsed = 0, 0.0
    with ThreadPoolExecutor(threads) as ex:
        t0 = time.perf_counter()
        while elapsed < budget_s:
            list(ex.map(one, work))
            reps += 1
            elapsed = time.perf_counter() - t0
    return reps, int(sum(int(x) for x in lens)) * reps, elapsed


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle on the headline batch (whole sequences, all heads):
    on all host threads (the reported value) and on one thread."""
    sh = case.shape
    threads = host_threads()
    reps, tokens_all, el_all = oracle_decode_parallel(case, budget_s / 4, threads)
    done, tokens, elapsed = oracle_decode_sample(case, budget_s)
    S = len(case.lengths)
    return {"value": reps * S / el_all, "unit": "tokens/s", "cores": threads,
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"the whole batch ({S} sequences, {tokens_all // reps} context tokens, all "
                      f"{sh.num_q_heads} heads) {reps} times, one sequence per task on "
                      f"{threads} threads, fp64, {el_all:.1f} s",
            "one_thread": {"value": done / elapsed, "unit": "tokens/s", "cores": 1,
                           "sample": f"{done} of {S} sequences ({tokens} context tokens), all "
                                     f"heads, fp64, {elapsed:.1f} s"}}


def cpu_decode_row(case, budget_s, tables=None, lengths=None, scales=(1.0, 1.0)):
    done, tokens, elapsed = oracle_decode_sample(case, budget_s, tables, lengths, scales)
    n = len(case.lengths if lengths is None else lengths)
    return {"value": done / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {n} sequences ({tokens} context tokens), all heads, fp64, "
                      f"one thread, {elapsed:.1f} s"}


def cpu_prefill_row(q, k_pool, v_pool, tables, cu, ctx, scale, block_size, budget_s,
                    scales=(1.0, 1.0)):
    """Oracle prefill on single rows of request 0 (each a 1-row chunk at its
    position, over all keys up to it) until the budget is spent.  ``scales``
    are the K and V cache scales of an fp8 pool."""
    oracle, gather_blocks, host_bits = _oracle_helpers()
    import numpy as np
    qlen0 = int(cu[1] - cu[0])
    done, elapsed = 0, 0.0
    for i in range(qlen0):
        pos = int(ctx[0]) - qlen0 + i
        k_sub, v_sub, t_sub, _ = gather_blocks(k_pool, v_pool, tables[:1], [pos + 1], [0],
                                               block_size)
        qrow = host_bits(q[int(cu[0]) + i:int(cu[0]) + i + 1])
        t0 = time.perf_counter()
        oracle.prefill(qrow, k_sub, v_sub, t_sub, np.array([0, 1], np.int32),
                       np.array([pos + 1], np.int32), scale, "bhrd", "bhdr",
                       k_scale=scales[0], v_scale=scales[1])
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= budget_s:
            break
    return {"value": done / elapsed, "unit": "query rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} query rows of request 0 (each over its >= {int(ctx[0]) - qlen0 + 1} "
                      f"visible keys), all heads, fp64, one thread, {elapsed:.1f} s"}


def cpu_cache_write_row(k_new, v_new, slots, hkv, d, bs, budget_s, fp8_scale=None):
    """Oracle cache write of the same tokens into a host pool holding just
    the blocks they touch, repeated until the budget is spent.  With
    ``fp8_scale`` the pools hold E4M3 codes and the write quantizes."""
    oracle, _, host_bits = _oracle_helpers()
    import numpy as np
    slots = np.asarray(slots, dtype=np.int64)
    blocks = np.unique(slots[slots >= 0] // bs)
    remap = {int(b): i for i, b in enumerate(blocks)}
    sub = np.array([remap[int(x) // bs] * bs + int(x) % bs if x >= 0 else -1 for x in slots],
                   dtype=np.int64)
    kh, vh = host_bits(k_new), host_bits(v_new)
    pool_dtype = kh.dtype if fp8_scale is None else np.uint8
    kp = np.zeros((len(blocks), hkv, bs, d), dtype=pool_dtype)
    vp = np.zeros((len(blocks), hkv, d, bs), dtype=pool_dtype)
    reps, elapsed = 0, 0.0
    while elapsed < budget_s:
        t0 = time.perf_counter()
        if fp8_scale is None:
            oracle.cache_write(kh, vh, kp, vp, sub, "bhrd", "bhdr")
        else:
            oracle.cache_write_fp8(kh, vh, kp, vp, sub, fp8_scale, fp8_scale, "bhrd", "bhdr")
        elapsed += time.perf_counter() - t0
        reps += 1
    return {"value": reps * len(slots) / elapsed, "unit": "tokens/s", "cores": 1,
            "kind": "oracle", "sample": f"{reps} writes of the {len(slots)} tokens into a host "
                                        f"pool of their {len(blocks)} blocks, {elapsed:.1f} s"}


def allocator_warm(pa, np, case, steps=300):
    """Warm host cost of one decode step's bookkeeping on the headline batch:
    a batch append of one token to each of the 64 sequences plus their dense
    tables, after 30 untimed steps.  `binding_us` goes through the Python
    binding; `c_abi_us` calls the two C entry points directly with the
    argument addresses bound once (the library's own cost)."""
    import ctypes
    sh = case.shape
    S = len(case.lengths)
    a = pa.Allocator(sh.num_blocks, sh.block_size, free_order=case.perm)
    ids = np.arange(S, dtype=np.int64)
    for s_ in ids:
        a.create(int(s_))
    a.batch_append(ids, case.lengths)
    stride = int(case.lengths.max() + 2 * steps + 100) // sh.block_size + 2
    ones = np.ones(S, dtype=np.int32)
    slots = np.zeros(S, dtype=np.int64)
    tabs = np.zeros((S, stride), dtype=np.int32)
    lens = np.zeros(S, dtype=np.int32)
    pad = sh.num_blocks - 1
    for _ in range(30):
        a.batch_append(ids, ones, slots_out=slots)
        a.batch_tables(ids, stride, pad, tables_out=tabs, lens_out=lens)
    t0 = time.perf_counter()
    for _ in range(steps):
        a.batch_append(ids, ones, slots_out=slots)
        a.batch_tables(ids, stride, pad, tables_out=tabs, lens_out=lens)
    binding = (time.perf_counter() - t0) * 1e6 / steps
    lib = pa.lib()
    pairs = np.zeros((S, 2), dtype=np.int32)
    n = ctypes.c_int32(0)
    app = (a._h, S, ids.ctypes.data, ones.ctypes.data, slots.ctypes.data, pairs.ctypes.data, S,
           ctypes.byref(n))
    tab = (a._h, S, ids.ctypes.data, tabs.ctypes.data, stride, pad, lens.ctypes.data)
    f_app, f_tab = lib.pa_batch_append, lib.pa_batch_tables
    t0 = time.perf_counter()
    for _ in range(steps):
        f_app(*app)
        f_tab(*tab)
    raw = (time.perf_counter() - t0) * 1e6 / steps
    return {"binding_us": binding, "c_abi_us": raw, "steps": steps, "stride": stride}


def cpu_allocator_row(case, steps):
    """The plain-Python reference model of the allocator replaying the
    headline batch's prompts and then `steps` decode appends of one token to
    every sequence, with the dense table built each step."""
    from oracle.allocator_model import AllocatorModel
    sh = case.shape
    m = AllocatorModel(sh.num_blocks, sh.block_size, free_order=case.perm)
    ids = list(range(len(case.lengths)))
    for s, L in zip(ids, case.lengths):
        m.create(s)
        m.append(s, int(L))
    t0 = time.perf_counter()
    for _ in range(steps):
        for s in ids:
            m.append(s, 1)
        [list(m.tables[s]) for s in ids]
    elapsed = time.perf_counter() - t0
    return {"value": elapsed * 1e6 / steps, "unit": "us/step", "cores": 1, "kind": "oracle",
            "sample": f"{steps} steps of 64 appends + tables on the Python reference model"}


def row_prefix_cache(pa, wl, np, cpu_budget):
    """Prefix cache on the chat workload: 128 requests opening with one of 16
    shared system prompts (2049..2063 tokens) plus 16..512 user tokens, block
    16, a 200,000-block shuffled pool.  Each request is admitted the way a
    scheduler would: reuse the cached full blocks of its prompt (leaving the
    last position to compute), then append the rest with token ids.  Host
    only: the kernels see ordinary block tables."""
    plan = wl.chat_plan()
    bs, nb = 16, 200_000
    order = np.random.default_rng(wl.SEED_BASE + 6).permutation(nb)
    prompts = [plan.prompt(r) for r in range(len(plan.user_tokens))]
    a = pa.Allocator(nb, bs, free_order=order)
    cached = 0
    t0 = time.perf_counter()
    for r, toks in enumerate(prompts):
        n = a.create_prefix(r, toks, len(toks) - 1)
        a.append_tokens(r, toks[n:])
        cached += n
    dt = time.perf_counter() - t0
    st = a.prefix_stats()
    total = sum(len(t) for t in prompts)
    out = {"host_us_per_request": dt * 1e6 / len(prompts),
           "hit_rate": st["hit_blocks"] / max(st["queried_blocks"], 1),
           "cached_token_frac": cached / total,
           "prefill_tokens_saved": cached, "prompt_tokens": total,
           "cached_blocks": st["cached_blocks"],
           "workload": "prefix cache: 128 requests over 16 shared system prompts of 2049..2063 "
                       "tokens + 16..512 user tokens, block 16, 200000-block pool (host, C ABI)"}
    if cpu_budget > 0:
        from oracle.allocator_model import AllocatorModel
        m = AllocatorModel(nb, bs, free_order=order)
        done, t0 = 0, time.perf_counter()
        for r, toks in enumerate(prompts):
            toks = toks.tolist()
            n = m.create_prefix(r, toks, len(toks) - 1)
            m.append(r, len(toks) - n, tokens=toks[n:])
            done += 1
            if time.perf_counter() - t0 > cpu_budget:
                break
        el = time.perf_counter() - t0
        out["cpu_oracle"] = {"value": el * 1e6 / done, "unit": "us/request", "cores": 1,
                             "kind": "oracle",
                             "sample": f"first {done} of {len(prompts)} requests on the Python "
                                       "reference model"}
    return out


def row_serving(pa, wl, torch, np, cpu_budget):
    """Continuous batching end to end: 256 requests (prompts U{128..2048},
    outputs U{16..256}) all queued at once, 7B-shaped attention geometry
    (32/32 heads, head_dim 128, block 16, bf16), a 16,384-block pool with a
    4,096-block pinned swap space, at most 128 running requests, 4,096 tokens
    and 1,024-token prompt chunks per step.  Each step: the C++ scheduler's
    plan, then swap/COW copies, the cache write of the new positions (N(0,1)
    rows), the prompt chunks and the decode batch on the GPU.  No model: the
    rate counts attention, cache and scheduling work only."""
    from paged_kv_cache_417_amd.driver import ServingLoop
    dev = "cuda"
    hq = hkv = 32
    d, bs = 128, 16
    rng = np.random.default_rng(wl.SEED_BASE + 8)
    n_req = 256
    prompts = rng.integers(128, 2048, n_req, endpoint=True)
    outs = rng.integers(16, 256, n_req, endpoint=True)
    loop = ServingLoop(num_blocks=16384, block_size=bs, num_q_heads=hq, num_kv_heads=hkv,
                       head_dim=d, max_num_seqs=128, max_batched_tokens=4096,
                       max_prefill_chunk=1024, max_context_len=2048 + 256, host_blocks=4096,
                       free_order=rng.permutation(16384))
    gen = wl.make_generator(wl.SEED_BASE + 8, dev)

    def rows(entries):
        n = sum(len(p) for _, p in entries)
        return (wl.randn((n, hkv, d), torch.bfloat16, gen, dev),
                wl.randn((n, hkv, d), torch.bfloat16, gen, dev))

    def qs(entries):
        return wl.randn((sum(len(p) for _, p in entries), hq, d), torch.bfloat16, gen, dev)

    for r in range(n_req):
        loop.add(r, int(prompts[r]), int(outs[r]))
    steps, dec_rows, pre_rows = 0, 0, 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while loop.sched.stats()["finished"] < n_req and steps < 5000:
        plan, _, _, _ = loop.step(rows, qs)
        steps += 1
        dec_rows += len(plan["decode"])
        pre_rows += sum(x[2] for x in plan["prefill"])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = loop.sched.stats()
    # host cost of the scheduler alone, replayed on a fresh allocator (no GPU work)
    a2 = pa.Allocator(16384, bs, free_order=np.random.default_rng(wl.SEED_BASE + 8).permutation(16384))
    a2.set_swap_space(4096)
    s2 = pa.Scheduler(a2, 128, 4096, 1024)
    for r in range(n_req):
        s2.add(r, int(prompts[r]), int(outs[r]))
    h0 = time.perf_counter()
    n2 = 0
    while s2.stats()["finished"] < n_req and n2 < 5000:
        s2.step()
        s2.complete()
        n2 += 1
    host_us = (time.perf_counter() - h0) * 1e6 / max(n2, 1)
    out = {"wall_s": wall, "steps": steps, "generated_tokens": int(outs.sum()),
           "prompt_tokens": int(prompts.sum()),
           "generated_tokens_per_s": int(outs.sum()) / wall,
           "prompt_tokens_per_s": int(prompts.sum()) / wall,
           "mean_decode_batch": dec_rows / max(steps, 1), "ms_per_step": wall * 1e3 / steps,
           "sched_host_us_per_step": host_us, "swap_preemptions": st["swap_preemptions"],
           "recompute_preemptions": st["recompute_preemptions"],
           "workload": "serving loop: 256 requests, prompts U[128,2048], outputs U[16,256], "
                       "7B-shaped attention (32/32 heads, D 128, block 16, bf16), 16384-block "
                       "pool + 4096 swap blocks, 128 seqs / 4096 tokens / 1024-token chunks per step"}
    if cpu_budget > 0:
        from oracle.allocator_model import AllocatorModel
        from oracle.scheduler_model import SchedulerModel
        m = AllocatorModel(16384, bs, free_order=np.random.default_rng(wl.SEED_BASE + 8).permutation(16384))
        m.set_swap_space(4096)
        ms = SchedulerModel(m, 128, 4096, 1024)
        for r in range(n_req):
            ms.add(r, int(prompts[r]), int(outs[r]))
        n3, t3 = 0, time.perf_counter()
        while ms.stats()["finished"] < n_req and time.perf_counter() - t3 < cpu_budget:
            ms.complete(ms.step())
            n3 += 1
        out["cpu_oracle"] = {"value": (time.perf_counter() - t3) * 1e6 / n3, "unit": "us/step",
                             "cores": 1, "kind": "oracle",
                             "sample": f"first {n3} scheduler steps on the Python reference model"}
    del loop
    return out


def row_serving_samples(pa, wl, torch, np):
    """Parallel sampling through the serving loop: 64 requests, each drawing 4
    samples from its prompt (prompts U{1024..2048}, outputs U{64..256} per
    sample), 7B-shaped attention (32/32 heads, head_dim 128, block 16, bf16),
    a 16,384-block pool, at most 128 sequences (32 requests), 4,096 tokens and
    1,024-token prompt chunks per step.  The scheduler forks each request's
    samples once its prompt is written.  The same request stream runs twice:
    decode batches grouped by request (pa_decode_grouped: the shared prompt
    blocks read once per group), then one sequence at a time (pa_decode with
    the cache-keeping policy).  Plans, and so all other work, are identical;
    every decode call is event-timed.  A short untimed pass warms up first."""
    from paged_kv_cache_417_amd.driver import ServingLoop
    dev = "cuda"
    hq = hkv = 32
    d, bs, nb, k = 128, 16, 16384, 4
    rng = np.random.default_rng(wl.SEED_BASE + 9)
    n_req = 64
    prompts = rng.integers(1024, 2048, n_req, endpoint=True)
    outs = rng.integers(64, 256, n_req, endpoint=True)
    order = rng.permutation(nb)
    out = {}
    # (False, True, False): the first pass warms up (first calls, allocator growth)
    for n_pass, grouped in enumerate((False, True, False)):
        n_run = 8 if n_pass == 0 else n_req
        loop = ServingLoop(num_blocks=nb, block_size=bs, num_q_heads=hq, num_kv_heads=hkv,
                           head_dim=d, max_num_seqs=128, max_batched_tokens=4096,
                           max_prefill_chunk=1024, max_context_len=2048 + 256,
                           free_order=order, group_samples=grouped)
        loop.time_decode = True
        gen = wl.make_generator(wl.SEED_BASE + 9, dev)

        def rows(entries):
            n = sum(len(p) for _, p in entries)
            return (wl.randn((n, hkv, d), torch.bfloat16, gen, dev),
                    wl.randn((n, hkv, d), torch.bfloat16, gen, dev))

        def qs(entries):
            return wl.randn((sum(len(p) for _, p in entries), hq, d), torch.bfloat16, gen, dev)

        for r in range(n_run):
            loop.add(r, int(prompts[r]), int(outs[r]),
                     samples=[100_000 + k * r + j for j in range(k - 1)])
        steps, dec_rows = 0, 0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while loop.sched.stats()["finished"] < n_run and steps < 5000:
            plan, _, _, _ = loop.step(rows, qs)
            steps += 1
            dec_rows += len(plan["decode"])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        dec_ms = loop.decode_ms()
        st = loop.sched.stats()
        if n_pass == 0:
            del loop
            continue
        key = "grouped" if grouped else "per_sequence"
        out[key] = {"wall_s": wall, "steps": steps, "ms_per_step": wall * 1e3 / steps,
                    "generated_tokens_per_s": k * int(outs.sum()) / wall,
                    "decode_ms_total": dec_ms, "decode_us_per_step": dec_ms * 1e3 / steps,
                    "mean_decode_batch": dec_rows / max(steps, 1),
                    "forked_samples": st["forked_samples"],
                    "swap_preemptions": st["swap_preemptions"],
                    "recompute_preemptions": st["recompute_preemptions"]}
        if grouped:
            out[key]["grouped_steps"] = loop.grouped_steps
            out[key]["mean_shared_blocks_per_step"] = loop.shared_block_reads / max(
                loop.grouped_steps, 1)
        del loop
        torch.cuda.empty_cache()
    out["speedup_wall"] = out["per_sequence"]["wall_s"] / out["grouped"]["wall_s"]
    out["speedup_decode"] = (out["per_sequence"]["decode_ms_total"] /
                             out["grouped"]["decode_ms_total"])
    out["workload"] = ("parallel sampling in the serving loop: 64 requests x 4 samples, prompts "
                       "U[1024,2048], outputs U[64,256] per sample, 7B-shaped attention (32/32 "
                       "heads, D 128, block 16, bf16), 16384-block pool, 128 seqs / 4096 tokens / "
                       "1024-token chunks per step; grouped (pa_decode_grouped per request) vs "
                       "per sequence (pa_decode, cache-keeping policy)")
    return out


PCIE_GBPS = 64.0  # PCIe 5.0 x16, per direction, nominal


def row_swap(pa, wl, torch, np, reps, cpu_budget):
    """Swap space: 8 sequences of 4096 tokens (7B-shaped blocks: 32 kv heads,
    head_dim 128, block 16, bf16; 256 KiB per block pair of K and V regions)
    move to a pinned host pool and back.  Each repetition is one swap-out of
    all eight (allocator + one pa_swap_blocks launch, device -> host) and one
    swap-in (host -> device); the copies are timed with HIP events."""
    dev = "cuda"
    hkv, d, bs, nb, nh = 32, 128, 16, 4096, 2048
    kshape, vshape = pa.kv_cache_shapes(nb, hkv, bs, d)
    k_dev = torch.empty(kshape, dtype=torch.bfloat16, device=dev)
    v_dev = torch.empty(vshape, dtype=torch.bfloat16, device=dev)
    gen = wl.make_generator(wl.SEED_BASE + 7, dev)
    for t in (k_dev, v_dev):  # content does not matter to the copy; fill it anyway
        for i in range(0, nb, 512):
            t[i:i + 512] = wl.randn(tuple(t[i:i + 512].shape), torch.bfloat16, gen, dev)
    hk, hv = pa.kv_cache_shapes(nh, hkv, bs, d)
    k_host = torch.empty(hk, dtype=torch.bfloat16, pin_memory=True)
    v_host = torch.empty(hv, dtype=torch.bfloat16, pin_memory=True)
    alloc = pa.Allocator(nb, bs, free_order=np.random.default_rng(wl.SEED_BASE + 7).permutation(nb))
    alloc.set_swap_space(nh)
    seqs = list(range(8))
    for sid in seqs:
        alloc.create(sid)
        alloc.append(sid, 4096)
    stream = torch.cuda.current_stream()
    t_out, t_in, host_us = [], [], []
    for rep in range(reps + 2):
        h0 = time.perf_counter()
        pairs = np.concatenate([alloc.swap_out(s) for s in seqs])
        h1 = time.perf_counter()
        dp = torch.as_tensor(pairs, device=dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        pa.pa_swap_blocks(k_dev, v_dev, k_host, v_host, dp)
        e[1].record(stream)
        h2 = time.perf_counter()
        pairs = np.concatenate([alloc.swap_in(s) for s in seqs])
        h3 = time.perf_counter()
        dp = torch.as_tensor(pairs, device=dev)
        e[2].record(stream)
        pa.pa_swap_blocks(k_host, v_host, k_dev, v_dev, dp)
        e[3].record(stream)
        torch.cuda.synchronize()
        if rep >= 2:  # two warm-ups
            t_out.append(e[0].elapsed_time(e[1]))
            t_in.append(e[2].elapsed_time(e[3]))
            host_us.append(((h1 - h0) + (h3 - h2)) * 1e6 / 2)
    n_pairs = len(pairs)
    moved = n_pairs * 2 * hkv * bs * d * 2
    mo, mi = sorted(t_out)[len(t_out) // 2], sorted(t_in)[len(t_in) // 2]
    out = {"us_out": mo * 1e3, "us_in": mi * 1e3, "bytes_each_way": moved,
           "GBps_out": moved / (mo * 1e-3) / 1e9, "GBps_in": moved / (mi * 1e-3) / 1e9,
           "frac_out_of_pcie5x16": moved / (mo * 1e-3) / 1e9 / PCIE_GBPS,
           "frac_in_of_pcie5x16": moved / (mi * 1e-3) / 1e9 / PCIE_GBPS,
           "host_us_per_swap_of_8": sorted(host_us)[len(host_us) // 2],
           "bound": "pcie",
           "workload": "swap 8 seqs x 4096 tokens (2048 blocks of 32 kv heads x 16 x 128 bf16, "
                       "K and V) to a pinned host pool and back"}
    if cpu_budget > 0:
        oracle, _, _ = _oracle_helpers()
        m = 64
        src_k = np.zeros((m, hkv, bs, d), np.uint16)
        src_v = np.zeros((m, hkv, d, bs), np.uint16)
        dst_k, dst_v = np.zeros_like(src_k), np.zeros_like(src_v)
        local = np.stack([np.arange(m), np.arange(m)[::-1]], axis=1).astype(np.int32)
        done, el = 0, 0.0
        while el < cpu_budget:
            t0 = time.perf_counter()
            oracle.swap_blocks(src_k, src_v, dst_k, dst_v, local, "bhrd", "bhdr")
            el += time.perf_counter() - t0
            done += m
        out["cpu_oracle"] = {"value": done * 2 * hkv * bs * d * 2 / el / 1e9, "unit": "GB/s",
                             "cores": 1, "kind": "oracle",
                             "sample": f"{done} block pairs copied host to host by the oracle"}
    del k_dev, v_dev, k_host, v_host
    return out


def cpu_copy_row(pairs, hkv, d, bs, budget_s):
    """Oracle whole-block copies of the same number of pairs on host pools."""
    oracle, _, _ = _oracle_helpers()
    import numpy as np
    n = len(pairs)
    kp = np.zeros((2 * n, hkv, bs, d), dtype=np.uint16)
    vp = np.zeros((2 * n, hkv, d, bs), dtype=np.uint16)
    local = np.stack([np.arange(n), np.arange(n, 2 * n)], axis=1).astype(np.int32)
    reps, elapsed = 0, 0.0
    while elapsed < budget_s:
        t0 = time.perf_counter()
        oracle.copy_blocks(kp, vp, local, "bhrd", "bhdr")
        elapsed += time.perf_counter() - t0
        reps += 1
    return {"value": reps * n / elapsed, "unit": "block pairs/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} copies of {n} block pairs (K and V, {hkv} heads) on host pools, "
                      f"{elapsed:.1f} s"}


# ---------------------------------------------------------------------------
# headline: 7B-shaped decode step


def headline(args, pa, wl, torch, np):
    """The 7B-shaped decode step, over R replicas of the batch (the same
    lengths in disjoint blocks of the pool, R = args.replicas): step i
    appends one token to every sequence of replica i mod R and decodes that
    replica, so each call reads K/V that the previous R - 1 calls did not
    touch (R x 2.2 GB between two reads of a block, against a 256 MB MALL)."""
    dev = "cuda"
    sh = wl.MHA_7B
    K, W = args.steps, args.warmup
    R = max(1, args.replicas)
    nsteps = K + W
    log(f"bench: building {sh.name} batch (S={sh.num_seqs} x {R} replicas, NB={sh.num_blocks})")
    host_steps = min(K, 20)
    grow = -(-(nsteps + host_steps + HOST_WARM) // R) + 1  # tokens a replica gains at most
    case = wl.make_decode_case(sh, dev, pa.K_AXES, pa.V_AXES, extra_table_slots=grow,
                               replicas=R)
    S = sh.num_seqs
    stride = case.tables.shape[1]
    pad = sh.num_blocks - 1

    # The allocator replays the prompts: with free_order = the batch's
    # permutation it hands out exactly the blocks the batch was laid into.
    alloc = pa.Allocator(sh.num_blocks, sh.block_size, free_order=case.perm)
    ids = np.arange(S * R, dtype=np.int64)
    for s in ids:
        alloc.create(int(s))
    alloc.batch_append(ids, case.lengths)
    t_chk, l_chk = alloc.batch_tables(ids, stride, pad)
    assert (t_chk == case.tables).all() and (l_chk == case.lengths).all()
    rep_ids = [ids[r * S:(r + 1) * S] for r in range(R)]

    # Every step's slots, tables and lengths, ahead of time (host cost timed).
    ones = np.ones(S, dtype=np.int32)
    h_slots = np.zeros((nsteps, S), dtype=np.int64)
    h_tabs = np.zeros((nsteps, S, stride), dtype=np.int32)
    h_lens = np.zeros((nsteps, S), dtype=np.int32)
    t0 = time.perf_counter()
    for i in range(nsteps):
        alloc.batch_append(rep_ids[i % R], ones, slots_out=h_slots[i])
        alloc.batch_tables(rep_ids[i % R], stride, pad, tables_out=h_tabs[i], lens_out=h_lens[i])
    alloc_us = (time.perf_counter() - t0) * 1e6 / nsteps
    d_slots = torch.as_tensor(h_slots, device=dev)
    d_tabs = torch.as_tensor(h_tabs, device=dev)
    d_lens = torch.as_tensor(h_lens, device=dev)

    gen = wl.make_generator(sh.seed + 1000, dev)
    k_new = wl.randn((nsteps, S, sh.num_kv_heads, sh.head_dim), torch.bfloat16, gen, dev)
    v_new = wl.randn((nsteps, S, sh.num_kv_heads, sh.head_dim), torch.bfloat16, gen, dev)
    q_all = wl.randn((nsteps, S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    out = torch.empty((S, sh.num_q_heads, sh.head_dim), device=dev)
    max_len = int(h_lens.max())
    ps = args.partition_size
    ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                             max_len, ps, dev)
    ps_used = ps or pa.pa_decode_default_partition(S, sh.num_kv_heads, sh.block_size, max_len)
    stream = torch.cuda.current_stream()
    # event pairs made before the loop; Python's garbage collector is off
    # while it runs (a collector pass between an event and its launch would
    # sit inside the event's interval)
    dec_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(K)]

    def step(i, timed):
        pa.pa_cache_write(k_new[i], v_new[i], case.k_pool, case.v_pool, d_slots[i])
        if timed:
            dec_events[i - W][0].record(stream)
        pa.pa_decode(out, q_all[i], case.k_pool, case.v_pool, d_tabs[i], d_lens[i], sh.scale,
                     max_len, ps, ws)
        if timed:
            dec_events[i - W][1].record(stream)

    log(f"bench: warmup {W} steps, partition {ps_used}")
    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    log(f"bench: timing {K} steps")
    gc_on = gc.isenabled()
    gc.disable()
    try:
        t0 = time.perf_counter()
        for i in range(W, nsteps):
            step(i, True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    finally:
        if gc_on:
            gc.enable()
    ms_step = (t1 - t0) * 1e3 / K
    dec_ms = [a.elapsed_time(b) for a, b in dec_events]
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    bytes_avg = sum(decode_bytes(h_lens[i], sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                                 sh.block_size) for i in range(W, nsteps)) / K
    achieved = bytes_avg / (dec_avg_ms * 1e-3) / 1e9
    assert torch.isfinite(out).all()
    log("bench: decode us per step: " + " ".join(f"{x * 1e3:.0f}" for x in dec_ms))
    log(f"bench: step {ms_step:.3f} ms, decode {dec_avg_ms * 1e3:.1f} us "
        f"(min {min(dec_ms) * 1e3:.1f}, max {max(dec_ms) * 1e3:.1f}), "
        f"{achieved:.0f} GB/s algorithmic, allocator {alloc_us:.1f} us/step on the host")

    # The same step with the host allocator and PCIe uploads inside the loop
    # (pinned staging, double-buffered); reported, never `value`.
    host_max = max_len + grow
    host_ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                                  host_max, ps, dev)
    host_rate = host_inclusive_rate(pa, wl, torch, np, case, alloc, rep_ids, stride, pad, k_new,
                                    v_new, q_all, out, host_ws, ps, host_max, host_steps)

    if args.calibrate:
        calibrate_copy(pa, torch, np, case, alloc)
    copy_ref = copy_reference(pa, torch, np, case, alloc, args.reps)
    read_ref = read_reference(pa, torch, case, args.reps)
    read_ref["decode_frac_of_read_stream"] = achieved / read_ref["GBps"]

    res = {
        "S": S, "replicas": R, "ms_step": ms_step, "dec_avg_ms": dec_avg_ms, "dec_ms": dec_ms,
        "bytes_avg": bytes_avg, "achieved": achieved, "ps": ps_used,
        "seq_len": float(h_lens[W:].mean()), "alloc_us": alloc_us, "host_rate": host_rate,
        "copy_ref": copy_ref, "read_ref": read_ref,
    }
    # the first replica as a batch of its own, for the CPU baseline
    first = wl.DecodeCase(sh, case.lengths[:S].copy(), case.perm, case.tables[:S].copy(),
                          case.q[:S], case.k_pool, case.v_pool, case.k_axes, case.v_axes)
    return first, res


def host_inclusive_rate(pa, wl, torch, np, case, alloc, rep_ids, stride, pad, k_new, v_new,
                        q_all, out, ws, ps, max_len, steps):
    """Decode steps with the host allocator and the uploads of slots, tables
    and lengths inside the loop (pinned staging, double-buffered), rotating
    over the replicas like the timed loop.  HOST_WARM untimed steps come
    first, and Python's garbage collector is off during the timed ones: one
    collector pass (tens of ms) inside 20 steps of ~0.4 ms would otherwise
    set the figure."""
    sh = case.shape
    S = len(rep_ids[0])
    R = len(rep_ids)
    dev = "cuda"
    h_slots = [torch.zeros(S, dtype=torch.int64).pin_memory() for _ in range(2)]
    h_tabs = [torch.zeros((S, stride), dtype=torch.int32).pin_memory() for _ in range(2)]
    h_lens = [torch.zeros(S, dtype=torch.int32).pin_memory() for _ in range(2)]
    d_slots = [torch.zeros(S, dtype=torch.int64, device=dev) for _ in range(2)]
    d_tabs = [torch.zeros((S, stride), dtype=torch.int32, device=dev) for _ in range(2)]
    d_lens = [torch.zeros(S, dtype=torch.int32, device=dev) for _ in range(2)]
    copied = [None, None]
    ones = np.ones(S, dtype=np.int32)
    stream = torch.cuda.current_stream()
    gc_on = gc.isenabled()
    gc.disable()
    try:
        t0 = None
        for i in range(-HOST_WARM, steps):
            if i == 0:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            b = i % 2
            if copied[b] is not None:
                copied[b].synchronize()
            ids = rep_ids[i % R]
            alloc.batch_append(ids, ones, slots_out=h_slots[b].numpy())
            alloc.batch_tables(ids, stride, pad, tables_out=h_tabs[b].numpy(),
                               lens_out=h_lens[b].numpy())
            d_slots[b].copy_(h_slots[b], non_blocking=True)
            d_tabs[b].copy_(h_tabs[b], non_blocking=True)
            d_lens[b].copy_(h_lens[b], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(stream)
            copied[b] = ev
            j = i % k_new.shape[0]
            pa.pa_cache_write(k_new[j], v_new[j], case.k_pool, case.v_pool, d_slots[b])
            pa.pa_decode(out, q_all[j], case.k_pool, case.v_pool, d_tabs[b], d_lens[b],
                         sh.scale, max_len, ps, ws)
        torch.cuda.synchronize()
        return S * steps / (time.perf_counter() - t0)
    finally:
        if gc_on:
            gc.enable()


def calibrate_copy(pa, torch, np, case, alloc):
    """One pa_copy_blocks launch over CALIB_PAIRS blocks nobody uses: reads
    and writes exactly CALIB_PAIRS * 2 * block_bytes each.  The counter runs
    divide the decode kernel's counters by this kernel's to calibrate."""
    st = alloc.stats()
    free = case.perm[st["num_used"]:-1]  # never handed out (the last entry is the pad block)
    assert len(free) >= 2 * CALIB_PAIRS
    pairs = np.stack([free[:CALIB_PAIRS], free[CALIB_PAIRS:2 * CALIB_PAIRS]], axis=1)
    d = torch.as_tensor(pairs.astype(np.int32), device="cuda")
    torch.cuda.synchronize()
    pa.pa_copy_blocks(case.k_pool, case.v_pool, d)
    torch.cuda.synchronize()
    log(f"bench: calibration copy of {CALIB_PAIRS} blocks done")


def copy_reference(pa, torch, np, case, alloc, reps):
    """A plain device copy on the same pool, as a second reference beside the
    8 TB/s peak: pa_copy_blocks over CALIB_PAIRS pairs of blocks that no
    sequence uses (K and V regions of 128 KiB each), 1 GiB read and 1 GiB
    written per call, event-timed."""
    st = alloc.stats()
    free = case.perm[st["num_used"]:-1]  # never handed out (the last entry is the pad block)
    pairs = np.stack([free[:CALIB_PAIRS], free[CALIB_PAIRS:2 * CALIB_PAIRS]], axis=1)
    d = torch.as_tensor(pairs.astype(np.int32), device="cuda")
    block_bytes = case.k_pool[0].numel() * case.k_pool.element_size()
    moved = CALIB_PAIRS * 2 * block_bytes  # read, and as many written
    stream = torch.cuda.current_stream()

    def call():
        pa.pa_copy_blocks(case.k_pool, case.v_pool, d)

    for _ in range(3):
        call()
    med, ms = events_time(torch, call, reps, stream)
    gbps = 2 * moved / (med * 1e-3) / 1e9
    return {"us": med * 1e3, **spread(ms), "bytes_read": moved, "bytes_written": moved,
            "GBps_read_plus_write": gbps, "frac_of_8TBps": gbps / PEAK_HBM_GBPS,
            "workload": f"pa_copy_blocks of {CALIB_PAIRS} unused block pairs of the headline pool "
                        f"(K and V, {block_bytes // 1024} KiB each)"}


READ_REF_BYTES = 8 << 30  # 32 times the MALL


def read_reference(pa, torch, case, reps):
    """The plain streaming read of the same GPU, as the practical ceiling
    beside the 8 TB/s peak: pa_read_stream over READ_REF_BYTES of the headline
    K pool (contiguous, 16-byte non-temporal loads, one XOR fold per
    workgroup), event-timed."""
    flat = case.k_pool.view(-1)
    n = min(flat.numel(), READ_REF_BYTES // flat.element_size())
    src = flat[:n]
    sink = torch.empty(pa.READ_STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        pa.pa_read_stream(src, sink)

    for _ in range(3):
        call()
    med, ms = events_time(torch, call, reps, stream)
    nbytes = n * flat.element_size()
    gbps = nbytes / (med * 1e-3) / 1e9
    return {"us": med * 1e3, **spread(ms), "bytes_read": nbytes, "GBps": gbps,
            "frac_of_8TBps": gbps / PEAK_HBM_GBPS,
            "workload": f"pa_read_stream over {nbytes >> 30} GiB of the headline K pool "
                        "(contiguous, 16-byte non-temporal loads)"}


# ---------------------------------------------------------------------------
# the other rows of the path, each on its own workload


ROTATE = 4  # disjoint copies of a decode batch visited in turn by the timed calls


def row_gqa(pa, wl, torch, np, reps, cpu_budget):
    sh = wl.GQA
    case = wl.make_decode_case(sh, "cuda", pa.K_AXES, pa.V_AXES, replicas=ROTATE)
    # the partition size the library picks from the batch's lengths (a
    # serving loop knows them on the host); the size-only default beside it
    S = sh.num_seqs
    ps = pa.decode_partition_for_lengths(case.lengths[:S], sh.num_kv_heads, sh.block_size,
                                         int(max(case.lengths)))
    r = decode_row(pa, torch, case, reps, ps=ps, replicas=ROTATE)
    r["partition_size"] = ps
    r["us_default_partition"] = decode_row(pa, torch, case, reps, replicas=ROTATE)["us"]
    if cpu_budget > 0:
        S = sh.num_seqs
        r["cpu_oracle"] = cpu_decode_row(case, cpu_budget, tables=case.tables[:S],
                                         lengths=case.lengths[:S])
    r["workload"] = ("gqa decode: 128 seqs, ctx round(lognormal(ln 1024, 1)) clipped "
                     "[16, 8192], 32 q / 8 kv heads, head_dim 128, block 16, bf16; "
                     "partitions of pa_decode_partition_for_lengths (us_default_partition: "
                     "pa_decode_default_partition's)")
    return r


def row_fp8(pa, wl, torch, np, reps, cpu_budget):
    """The 7B-shaped decode batch (same lengths, tables and pool size) with an
    fp8 (OCP E4M3) K/V cache, one scale per cache: half the K/V bytes."""
    sh = wl.DecodeShape("mha_7b", 64, 32, 32, 128, 16, 200_000, "fp8", wl.MHA_7B.seed)
    case = wl.make_decode_case(sh, "cuda", pa.K_AXES, pa.V_AXES, replicas=ROTATE)

    def dec(out, q, k, v, t, l, maxlen, ps, ws):
        pa.pa_decode_fp8(out, q, k, v, t, l, sh.scale, wl.FP8_SCALE, wl.FP8_SCALE, maxlen, ps,
                         ws)

    r = decode_row(pa, torch, case, reps, replicas=ROTATE, decode=dec)
    r["workload"] = ("7B-shaped decode with fp8 (E4M3) K/V: 64 seqs, ctx U[128,4096], 32/32 "
                     "heads, head_dim 128, block 16, 200000-block pool, one scale per cache")
    if cpu_budget > 0:
        S = sh.num_seqs
        r["cpu_oracle"] = cpu_decode_row(case, cpu_budget, tables=case.tables[:S],
                                         lengths=case.lengths[:S],
                                         scales=(wl.FP8_SCALE, wl.FP8_SCALE))
    return r


def row_mha_valu(pa, wl, torch, np, reps):
    """The 7B-shaped decode batch on the vector-ALU kernel (PA_DECODE_VALU),
    rotated like the headline: the A/B of the matrix-core choice for MHA."""
    sh = wl.MHA_7B
    case = wl.make_decode_case(sh, "cuda", pa.K_AXES, pa.V_AXES, replicas=ROTATE)

    def dec(out, q, k, v, t, l, maxlen, ps, ws):
        pa.pa_decode(out, q, k, v, t, l, sh.scale, maxlen, ps, ws, valu=True)

    r = decode_row(pa, torch, case, reps, replicas=ROTATE, decode=dec)
    r_mfma = decode_row(pa, torch, case, reps, replicas=ROTATE)
    r["matrix_core_kernel_us"] = r_mfma["us"]
    r["workload"] = ("7B-shaped decode (64 seqs, ctx U[128,4096], 32/32 heads, head_dim 128, "
                     "block 16, bf16) on the vector-ALU kernel; matrix_core_kernel_us: the "
                     "default kernel on the same calls")
    return r


def row_long(pa, wl, torch, np, reps, cpu_budget):
    """8 x 32768 tokens at block 128: the library's default partitions (the
    row's figure) and the 512-token partitions the long-context workload
    names, beside it.  Four copies need 8192 blocks, so the pool holds 8320."""
    sh = wl.MIXED_DECODE
    case = wl.make_decode_case(sh, "cuda", pa.K_AXES, pa.V_AXES, replicas=ROTATE,
                               num_blocks=ROTATE * 2048 + 128)
    S = sh.num_seqs
    ps = pa.pa_decode_default_partition(S, sh.num_kv_heads, sh.block_size,
                                        int(case.lengths.max()))
    r = decode_row(pa, torch, case, reps, ps=sh.partition_size, replicas=ROTATE)
    r512 = decode_row(pa, torch, case, reps, ps=512, replicas=ROTATE)
    r["at_512_token_partitions"] = {k: r512[k] for k in ("us", "p10_us", "p90_us", "GBps",
                                                         "frac_of_8TBps")}
    if cpu_budget > 0:
        r["cpu_oracle"] = cpu_decode_row(case, cpu_budget, tables=case.tables[:S],
                                         lengths=case.lengths[:S])
    r["workload"] = ("long-context split-K decode: 8 seqs x 32768 tokens, block 128, "
                     f"partitions of {ps} (library default; 512 beside it), 32 q / 8 kv heads, "
                     "head_dim 128, bf16")
    return r


def decode_row(pa, torch, case, reps, ps=0, tables=None, lengths=None, kv_reuse=False,
               groups=None, max_group=0, replicas=1, decode=None):
    """Event-timed decode calls on one workload.  With replicas > 1 the case
    holds that many copies of the batch in disjoint blocks (sequences r*S ..
    r*S+S-1) and call k decodes copy k mod replicas, so no call re-reads
    what the previous ones read.  decode: the call to time (pa.pa_decode by
    default), given (out, q, k_pool, v_pool, tables, lens, maxlen, ps, ws)."""
    sh = case.shape
    dev = "cuda"
    lens = case.lengths if lengths is None else lengths
    tabs = case.tables if tables is None else tables
    S = len(lens) // replicas
    maxlen = int(max(lens))
    t_dev = [torch.as_tensor(tabs[r * S:(r + 1) * S], device=dev) for r in range(replicas)]
    l_dev = [torch.as_tensor(lens[r * S:(r + 1) * S], device=dev) for r in range(replicas)]
    q_rep = [case.q[r * S:(r + 1) * S] for r in range(replicas)]
    out = torch.empty((S, sh.num_q_heads, sh.head_dim), device=dev)
    ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                             maxlen, ps, dev, grouped=groups is not None)
    stream = torch.cuda.current_stream()

    if groups is not None:
        g_dev = [torch.as_tensor(a, device=dev) for a in groups]
    k = [0]

    def call():
        r = k[0] % replicas
        k[0] += 1
        if decode is not None:
            decode(out, q_rep[r], case.k_pool, case.v_pool, t_dev[r], l_dev[r], maxlen, ps, ws)
        elif groups is None:
            pa.pa_decode(out, q_rep[r], case.k_pool, case.v_pool, t_dev[r], l_dev[r], sh.scale,
                         maxlen, ps, ws, kv_reuse=kv_reuse)
        else:
            pa.pa_decode_grouped(out, q_rep[r], case.k_pool, case.v_pool, t_dev[r], l_dev[r],
                                 sh.scale, maxlen, g_dev[0], g_dev[1], g_dev[2], max_group, ps,
                                 ws, kv_reuse=kv_reuse)

    for _ in range(max(3, replicas)):
        call()
    med, all_ms = events_time(torch, call, reps, stream)
    e_kv = 1 if case.k_pool.dtype == torch.uint8 else 2
    b = decode_bytes(lens[:S], sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                     e_kv=e_kv)
    gbps = b / (med * 1e-3) / 1e9
    r = {"us": med * 1e3, **spread(all_ms), "algorithmic_bytes": b, "GBps": gbps,
         "frac_of_8TBps": gbps / PEAK_HBM_GBPS, "tokens_per_s": S / (med * 1e-3),
         "bound": "hbm"}
    if replicas > 1:
        r["rotation"] = (f"{replicas} copies of the batch in disjoint blocks, visited in turn "
                         f"({replicas * b / 1e9:.2f} GB between two reads of a block)")
    return r


def prefix_shared_batch(pa, wl, torch, np, before_tails=None):
    """The prefix-shared batch: 16 prompts of 2048 + j tokens, each forked
    into 8 samples; the samples' first appends copy the shared partial block
    (112 copies), then their tails are written.  before_tails(k_pool,
    v_pool, pairs_on_device) runs between the copies and the tail writes.
    Returns (case, alloc, pairs, append_us, samples)."""
    sh = wl.PREFIX_SHARED
    dev = "cuda"
    plan = wl.prefix_plan()
    rng = np.random.default_rng(sh.seed)
    order = rng.permutation(sh.num_blocks)
    alloc = pa.Allocator(sh.num_blocks, sh.block_size, free_order=order)
    kshape, vshape = pa.kv_cache_shapes(sh.num_blocks, sh.num_kv_heads, sh.block_size,
                                        sh.head_dim)
    k_pool = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
    gen = wl.make_generator(sh.seed, dev)
    n_prompts, samples = plan.tail_lens.shape
    pids = [1000 * i for i in range(n_prompts)]
    for p in pids:
        alloc.create(p)
    slots, _ = alloc.batch_append(pids, plan.shared_lens)
    shape = (len(slots), sh.num_kv_heads, sh.head_dim)
    pa.pa_cache_write(wl.randn(shape, torch.bfloat16, gen, dev),
                      wl.randn(shape, torch.bfloat16, gen, dev), k_pool, v_pool,
                      torch.as_tensor(slots, device=dev))
    ids = []
    for p in pids:
        ids.append(p)
        for k in range(1, samples):
            alloc.fork(p, p + k)
            ids.append(p + k)
    t0 = time.perf_counter()
    slots, pairs = alloc.batch_append(ids, plan.tail_lens.reshape(-1))
    append_us = (time.perf_counter() - t0) * 1e6
    d_pairs = torch.as_tensor(pairs, device=dev)
    pa.pa_copy_blocks(k_pool, v_pool, d_pairs)
    if before_tails is not None:
        before_tails(k_pool, v_pool, d_pairs)
    shape = (len(slots), sh.num_kv_heads, sh.head_dim)
    pa.pa_cache_write(wl.randn(shape, torch.bfloat16, gen, dev),
                      wl.randn(shape, torch.bfloat16, gen, dev), k_pool, v_pool,
                      torch.as_tensor(slots, device=dev))
    stride = max(wl.blocks_needed(alloc.length(s), sh.block_size) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    q = wl.randn((len(ids), sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    case = wl.DecodeCase(sh, lens, order, tables, q, k_pool, v_pool, pa.K_AXES, pa.V_AXES)
    return case, alloc, pairs, append_us, samples


def row_prefix_shared(pa, wl, torch, np, reps, cpu_budget):
    """16 prompts x 8 samples sharing the prompt's blocks; 112 copy-on-writes
    of the partial shared block before the tails are written."""
    sh = wl.PREFIX_SHARED
    stream = torch.cuda.current_stream()
    copy_ms = []

    def time_copy(k_pool, v_pool, d_pairs):
        def copy():
            pa.pa_copy_blocks(k_pool, v_pool, d_pairs)
        # idempotent before the tails are written: the sources are unchanged
        copy_ms.append(events_time(torch, copy, reps, stream)[0])

    case, alloc, pairs, append_us, samples = prefix_shared_batch(pa, wl, torch, np, time_copy)
    copy_med = copy_ms[0]
    block_bytes = sh.num_kv_heads * sh.block_size * sh.head_dim * 2
    copy_bytes = len(pairs) * 2 * block_bytes * 2  # K and V regions, read + write
    tables, lens, ids = case.tables, case.lengths, range(len(case.lengths))
    # The allocator reports shared blocks: the batch is decoded with the
    # samples of each prompt as one group (pa_decode_grouped: the shared
    # region is read once per group) at the partition size
    # pa_decode_grouped_partition picks, with the streaming load policy (no
    # block is read twice).  The grouped call at the plain default size and
    # the per-sequence decode with the cache-keeping policy (the sharers'
    # re-reads hit the caches) and the streaming one are timed beside it.
    assert alloc.stats()["num_shared"] > 0
    maxlen = int(lens.max())
    ps0 = pa.pa_decode_default_partition(len(ids), sh.num_kv_heads, sh.block_size, maxlen)
    groups = pa.decode_groups(tables, lens, np.arange(len(ids)) // samples, sh.block_size)
    ps = pa.decode_grouped_partition(lens, *groups, sh.num_q_heads, sh.num_kv_heads,
                                     sh.block_size, maxlen)
    groups = groups[:3]
    r = decode_row(pa, torch, case, reps, ps=ps, groups=groups, max_group=samples)
    r["partition_size"] = ps
    r["us_grouped_default_partition"] = decode_row(pa, torch, case, reps, ps=ps0, groups=groups,
                                                   max_group=samples)["us"]
    r["us_per_sequence"] = decode_row(pa, torch, case, reps, kv_reuse=True)["us"]
    r["us_streaming_policy"] = decode_row(pa, torch, case, reps)["us"]
    r["shared_partitions_per_group"] = -(-int(groups[2][0]) * sh.block_size // ps)
    # unique bytes: each physical block's valid rows once
    unique_tokens = 0
    seen = set()
    for s in range(len(ids)):
        for j in range(wl.blocks_needed(int(lens[s]), sh.block_size)):
            b = int(tables[s, j])
            if b not in seen:
                seen.add(b)
                unique_tokens += min(sh.block_size, int(lens[s]) - j * sh.block_size)
    kv_unique = unique_tokens * sh.num_kv_heads * sh.head_dim * 2 * 2
    kv_logical = int(lens.sum()) * sh.num_kv_heads * sh.head_dim * 2 * 2
    other = r["algorithmic_bytes"] - kv_logical
    r["unique_bytes"] = kv_unique + other
    r["GBps_unique"] = r["unique_bytes"] / (r["us"] * 1e-6) / 1e9
    r["frac_unique_of_8TBps"] = r["GBps_unique"] / PEAK_HBM_GBPS
    # logical bytes count every sharer's read of a shared block: a rate, not
    # a fraction of the HBM peak
    r["GBps_logical"] = r.pop("GBps")
    r.pop("frac_of_8TBps")
    r["logical_bytes"] = r.pop("algorithmic_bytes")
    r["workload"] = ("prefix-shared decode: 16 prompts of 2048+j tokens x 8 samples sharing "
                     "them, tails U[1,512], 32/32 heads, head_dim 128, block 16, bf16; us: "
                     "pa_decode_grouped (one group per prompt, pa_decode_grouped_partition's "
                     "size, streaming policy), us_per_sequence: pa_decode_ex with the "
                     "cache-keeping policy")
    if cpu_budget > 0:
        r["cpu_oracle"] = cpu_decode_row(case, cpu_budget)
    cow = {"us": copy_med * 1e3, "pairs": int(len(pairs)), "bytes_moved": copy_bytes,
           "GBps": copy_bytes / (copy_med * 1e-3) / 1e9, "bound": "latency (256 KiB per pair)",
           "host_append_us": append_us,
           "workload": "copy-on-write of the 112 shared partial blocks (K+V, 32 heads)"}
    cow["gpu_block_pairs_per_s"] = len(pairs) / (copy_med * 1e-3)
    if cpu_budget > 0:
        cow["cpu_oracle"] = cpu_copy_row(pairs, sh.num_kv_heads, sh.head_dim, sh.block_size,
                                         cpu_budget)
    return r, cow


def row_mixed(pa, wl, torch, np, reps, cpu_budget):
    """Mixed step: 8 decode sequences at 32768 tokens and 4 prompt chunks of
    512 new tokens over 4096 cached, one cache write for all 2056 new rows."""
    dev = "cuda"
    dsh, psh = wl.MIXED_DECODE, wl.MIXED_PREFILL
    hkv, d, bs = dsh.num_kv_heads, dsh.head_dim, dsh.block_size
    nb = dsh.num_blocks
    rng = np.random.default_rng(dsh.seed)
    alloc = pa.Allocator(nb, bs, free_order=rng.permutation(nb))
    dec_ids, pre_ids = list(range(8)), list(range(100, 104))
    for s in dec_ids + pre_ids:
        alloc.create(s)
    kshape, vshape = pa.kv_cache_shapes(nb, hkv, bs, d)
    k_pool = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
    gen = wl.make_generator(dsh.seed, dev)
    slots, _ = alloc.batch_append(dec_ids + pre_ids, [32767] * 8 + [4096] * 4)
    for lo in range(0, len(slots), 65536):
        hi = min(len(slots), lo + 65536)
        shape = (hi - lo, hkv, d)
        pa.pa_cache_write(wl.randn(shape, torch.bfloat16, gen, dev),
                          wl.randn(shape, torch.bfloat16, gen, dev), k_pool, v_pool,
                          torch.as_tensor(slots[lo:hi], device=dev))
    slots, _ = alloc.batch_append(dec_ids + pre_ids, [1] * 8 + [512] * 4)
    d_slots = torch.as_tensor(slots, device=dev)
    kn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    vn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    dt, dl = alloc.batch_tables(dec_ids, 257)
    pt, pl = alloc.batch_tables(pre_ids, 40)
    dt, dl, pt, pl = (torch.as_tensor(x, device=dev) for x in (dt, dl, pt, pl))
    cu = torch.as_tensor(np.arange(0, 2049, 512, dtype=np.int32), device=dev)
    qd = wl.randn((8, dsh.num_q_heads, d), torch.bfloat16, gen, dev)
    qp = wl.randn((2048, psh.num_q_heads, d), torch.bfloat16, gen, dev)
    out_d = torch.empty((8, dsh.num_q_heads, d), device=dev)
    out_p = torch.empty((2048, psh.num_q_heads, d), device=dev)
    ws = pa.decode_workspace(8, dsh.num_q_heads, hkv, d, bs, 32768, dsh.partition_size, dev)
    stream = torch.cuda.current_stream()

    def cw():
        pa.pa_cache_write(kn, vn, k_pool, v_pool, d_slots)

    def dec():
        pa.pa_decode(out_d, qd, k_pool, v_pool, dt, dl, dsh.scale, 32768, dsh.partition_size, ws)

    def pre():
        pa.pa_prefill_chunk(out_p, qp, k_pool, v_pool, pt, cu, pl, psh.scale, 512, 4608)

    def step():
        cw()
        dec()
        pre()

    for f in (cw, dec, pre, step):
        f()
    cw_med, _ = events_time(torch, cw, reps, stream)
    warm(torch, pre, 1.0)
    pre_med, pre_ms = events_time(torch, pre, reps, stream)
    step_med, _ = events_time(torch, step, reps, stream)
    flops = prefill_flops([4608] * 4, [512] * 4, psh.num_q_heads, d)
    cw_bytes = len(slots) * hkv * d * 2 * 2 * 2  # K and V rows, read + write
    prefill = {"us": pre_med * 1e3, **spread(pre_ms), "flops": flops,
               "TFLOPs": flops / (pre_med * 1e-3) / 1e12,
               "frac_of_2.5PF_bf16": flops / (pre_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "bound": "mfma",
               "workload": "chunked prefill: 4 requests x 512 new tokens over 4096 cached "
                           "(causal), 32 q / 8 kv heads, head_dim 128, block 128, bf16"}
    cache_write = {"us": cw_med * 1e3, "tokens": len(slots), "bytes_moved": cw_bytes,
                   "GBps": cw_bytes / (cw_med * 1e-3) / 1e9, "bound": "latency",
                   "workload": "cache write of 8 decode + 2048 prompt-chunk tokens, 8 kv heads, "
                               "head_dim 128, block 128, bf16"}
    prefill["gpu_query_rows_per_s"] = 2048 / (pre_med * 1e-3)
    cache_write["gpu_tokens_per_s"] = len(slots) / (cw_med * 1e-3)
    if cpu_budget > 0:
        torch.cuda.synchronize()
        prefill["cpu_oracle"] = cpu_prefill_row(qp, k_pool, v_pool, pt.cpu().numpy(),
                                                cu.cpu().numpy(), pl.cpu().numpy(), psh.scale,
                                                bs, cpu_budget)
        cache_write["cpu_oracle"] = cpu_cache_write_row(kn, vn, slots, hkv, d, bs, cpu_budget)
    mixed = {"us": step_med * 1e3,
             "workload": "cache write (2056 tokens) + decode 8 x 32768 (split-K, default partitions) + "
                         "prefill 4 x 512 over 4096, one stream"}
    return prefill, cache_write, mixed


def row_fp8_prefill(pa, wl, torch, np, reps, cpu_budget):
    """The mixed step's prompt chunks (4 requests x 512 new tokens over 4096
    cached, causal) over E4M3 caches: the quantizing write of the chunks' 2048
    K/V rows and the chunked prefill that reads the pool."""
    dev = "cuda"
    psh = wl.PrefillShape(dtype="fp8")
    case = wl.make_prefill_case(psh, dev, pa.K_AXES, pa.V_AXES)
    hkv, d, bs = psh.num_kv_heads, psh.head_dim, psh.block_size
    R, new, ctx = psh.num_reqs, psh.new_tokens, case.context_lens
    slots = np.concatenate([
        case.tables[r][np.arange(ctx[r] - new, ctx[r]) // bs].astype(np.int64) * bs
        + np.arange(ctx[r] - new, ctx[r]) % bs for r in range(R)])
    gen = wl.make_generator(psh.seed + 1, dev)
    kn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    vn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    d_slots = torch.as_tensor(slots, device=dev)
    t_dev = torch.as_tensor(case.tables, device=dev)
    cu = torch.as_tensor(case.cu_q_lens, device=dev)
    cl = torch.as_tensor(ctx, device=dev)
    tq = int(case.cu_q_lens[-1])
    out = torch.empty((tq, psh.num_q_heads, d), device=dev)
    stream = torch.cuda.current_stream()
    sc = wl.FP8_SCALE

    def cw():
        pa.pa_cache_write_fp8(kn, vn, case.k_pool, case.v_pool, d_slots, sc, sc)

    def pre():
        pa.pa_prefill_chunk_fp8(out, case.q, case.k_pool, case.v_pool, t_dev, cu, cl, psh.scale,
                                sc, sc, new, int(ctx.max()))

    for f in (cw, pre):
        f()
    cw_med, _ = events_time(torch, cw, reps, stream)
    warm(torch, pre, 1.0)
    pre_med, pre_ms = events_time(torch, pre, reps, stream)
    flops = prefill_flops([int(c) for c in ctx], [new] * R, psh.num_q_heads, d)
    cw_bytes = len(slots) * hkv * d * (2 + 1) * 2  # bf16 rows in, E4M3 codes out, K and V
    prefill = {"us": pre_med * 1e3, **spread(pre_ms), "flops": flops,
               "TFLOPs": flops / (pre_med * 1e-3) / 1e12,
               "frac_of_2.5PF_bf16": flops / (pre_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
               "bound": "mfma (bf16 products after widening the codes)",
               "gpu_query_rows_per_s": tq / (pre_med * 1e-3),
               "workload": "chunked prefill over an fp8 (E4M3) cache: 4 requests x 512 new "
                           "tokens over 4096 cached (causal), 32 q / 8 kv heads, head_dim 128, "
                           "block 128, one scale per cache, bf16 q"}
    cache_write = {"us": cw_med * 1e3, "tokens": len(slots), "bytes_moved": cw_bytes,
                   "GBps": cw_bytes / (cw_med * 1e-3) / 1e9, "bound": "latency",
                   "gpu_tokens_per_s": len(slots) / (cw_med * 1e-3),
                   "workload": "quantizing cache write of the 2048 prompt-chunk rows (bf16 in, "
                               "E4M3 out), 8 kv heads, head_dim 128, block 128"}
    if cpu_budget > 0:
        torch.cuda.synchronize()
        prefill["cpu_oracle"] = cpu_prefill_row(case.q, case.k_pool, case.v_pool, case.tables,
                                                case.cu_q_lens, ctx, psh.scale, bs, cpu_budget,
                                                scales=(sc, sc))
        # The oracle's E4M3 encode searches the code table: 512 of the tokens
        # keep one repetition near a second.
        cache_write["cpu_oracle"] = cpu_cache_write_row(kn[:512], vn[:512], slots[:512], hkv, d,
                                                        bs, cpu_budget, fp8_scale=sc)
    return prefill, cache_write


# ---------------------------------------------------------------------------
# counter summaries


def _read_counters(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, kernel_substr):
    """Counter totals per dispatch of the kernels whose names contain
    kernel_substr (a string, or a tuple of alternatives)."""
    subs = (kernel_substr,) if isinstance(kernel_substr, str) else tuple(kernel_substr)
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name", "")
        if r.get("Counter_Name") != counter or not any(k in name for k in subs):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    return list(acc.values())


def pmc_summary(fetch_dir, write_dir, block_bytes):
    """Per-launch HBM bytes of the decode kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by the same counter's reading for the
    calibration copy (CALIB_PAIRS blocks of block_bytes per K and V region,
    read once and written once)."""
    expect = CALIB_PAIRS * 2 * block_bytes
    out = {"kernel": " or ".join(DECODE_KERNEL), "kernel_source_sha256": kernel_source_hash(),
           "calibration": f"pa_copy_blocks over {CALIB_PAIRS} blocks: {expect} B read, "
                          f"{expect} B written"}
    total = 0.0
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_counters(d)
        dec = _per_dispatch(rows, name, DECODE_KERNEL)
        cal = _per_dispatch(rows, name, "copy_blocks_kernel")
        cal = [c for c in cal if c * 1024 > expect / 4]  # the calibration launch, not COW copies
        if not dec or not cal:
            raise SystemExit(f"{name}: decode dispatches {len(dec)}, calibration {len(cal)}")
        factor = expect / (sum(cal) / len(cal) * 1024)
        per_launch = sum(dec) / len(dec) * 1024 * factor
        out[name] = {"decode_kib_per_dispatch_raw": sum(dec) / len(dec),
                     "calibration_kib_raw": sum(cal) / len(cal), "scale": factor,
                     "decode_bytes_per_launch": per_launch, "dispatches": len(dec)}
        total += per_launch
    out["hbm_bytes_per_launch"] = total
    return out


NUM_CUS = 256  # MI355X
NUM_SIMDS = NUM_CUS * 4
NUM_XCCS = 8


def prefill_only(pa, wl, torch, reps):
    """The mixed step's prompt chunks alone (4 x 512 new tokens over 4096
    cached, bf16 and fp8 caches): `reps` timed calls each, for the counter
    runs.  Prints one JSON line."""
    out = {}
    for dtype in ("bf16", "fp8"):
        psh = wl.PrefillShape(dtype=dtype)
        case = wl.make_prefill_case(psh, "cuda", pa.K_AXES, pa.V_AXES)
        t_dev = torch.as_tensor(case.tables, device="cuda")
        cu = torch.as_tensor(case.cu_q_lens, device="cuda")
        cl = torch.as_tensor(case.context_lens, device="cuda")
        mx = int(case.context_lens.max())
        o = torch.empty((int(case.cu_q_lens[-1]), psh.num_q_heads, psh.head_dim), device="cuda")

        def call():
            if dtype == "fp8":
                pa.pa_prefill_chunk_fp8(o, case.q, case.k_pool, case.v_pool, t_dev, cu, cl,
                                        psh.scale, wl.FP8_SCALE, wl.FP8_SCALE, psh.new_tokens, mx)
            else:
                pa.pa_prefill_chunk(o, case.q, case.k_pool, case.v_pool, t_dev, cu, cl,
                                    psh.scale, psh.new_tokens, mx)

        warm(torch, call, 1.0)
        med, all_ms = events_time(torch, call, reps, torch.cuda.current_stream())
        flops = prefill_flops([int(c) for c in case.context_lens],
                              [psh.new_tokens] * psh.num_reqs, psh.num_q_heads, psh.head_dim)
        out[dtype] = {"us": med * 1e3, "TFLOPs": flops / (med * 1e-3) / 1e12, "flops": flops}
        del case
        torch.cuda.empty_cache()
    print(json.dumps({"prefill_only": out}), flush=True)


def prefill_counter_summary(dirs):
    """Markdown table of SQ counters per prefill dispatch (bf16 and fp8 cache
    instantiations) from rocprofv3 --pmc runs, with the matrix-core busy share
    (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs, rocprof's MfmaUtil)
    and the vector-ALU busy share (SQ_ACTIVE_INST_VALU over GRBM_GUI_ACTIVE x
    CUs, rocprof's VALUBusy)."""
    rows = []
    for i, d in enumerate(dirs):
        rows += [dict(r, run=i) for r in _read_counters(d)]
    per = {}
    for r in rows:
        name = r.get("Kernel_Name", "")
        if "prefill_kernel<128, 128, " in name:  # demangled
            kind = "fp8" if "prefill_kernel<128, 128, true>" in name else "bf16"
        elif "prefill_kernelILi128ELi128ELb" in name:  # mangled: ...ELb1E = fp8
            kind = "fp8" if "prefill_kernelILi128ELi128ELb1E" in name else "bf16"
        else:
            continue
        key = (kind, r.get("Counter_Name"))
        disp = (r["run"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        per.setdefault(key, {}).setdefault(disp, 0.0)
        per[key][disp] += float(r["Counter_Value"])
    lines = ["| cache | counter | mean per dispatch | dispatches |", "|---|---|---|---|"]
    means = {}
    for (kind, c), v in sorted(per.items()):
        m = sum(v.values()) / len(v)
        means[(kind, c)] = m
        lines.append(f"| {kind} | {c} | {m:.4g} | {len(v)} |")
    lines.append("")
    for kind in ("bf16", "fp8"):
        g = means.get((kind, "GRBM_GUI_ACTIVE"))
        if not g:
            continue
        # the csv sums the counter over the 8 XCCs; each counts the same clock
        g /= NUM_XCCS
        lines.append(f"- {kind}: {g:.4g} GPU cycles per dispatch (GRBM_GUI_ACTIVE / {NUM_XCCS})")
        mf = means.get((kind, "SQ_VALU_MFMA_BUSY_CYCLES"))
        va = means.get((kind, "SQ_ACTIVE_INST_VALU"))
        if mf is not None:
            lines.append(f"- {kind}: matrix core busy {100 * mf / (g * NUM_SIMDS):.1f}% "
                         f"(rocprof's MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles))")
        if va is not None:
            lines.append(f"- {kind}: vector ALU busy {100 * va / (g * NUM_CUS):.1f}% "
                         f"(rocprof's VALUBusy: SQ_ACTIVE_INST_VALU / (CUs x cycles))")
    return "\n".join(lines)


CAL_PHASE = "calibration copy"
DECODE_PHASES = ("7B-shaped decode (rotated)", "gqa decode (rotated)", "fp8 decode (rotated)",
                 "long-context decode, default partitions (rotated)",
                 "long-context decode, 512-token partitions (rotated)",
                 "prefix-shared grouped decode", CAL_PHASE,
                 "7B-shaped decode on the vector-ALU kernel (rotated)")


def decode_only(pa, wl, torch, np, reps, out_json):
    """Every decode workload alone, for the counter runs: `reps` pa_decode
    calls per workload (four disjoint copies of each batch visited in turn,
    except the prefix-shared one), each workload after a spin-kernel marker,
    then the calibration copy.  Writes each phase's algorithmic bytes per
    call to out_json."""
    dev = "cuda"
    phases = []

    def run(name, case, ps=0, replicas=ROTATE, **kw):
        mark_phase(torch)
        r = decode_row(pa, torch, case, reps, ps=ps, replicas=replicas, **kw)
        phases.append({"phase": name, "algorithmic_bytes": r.get("algorithmic_bytes",
                                                                 r.get("unique_bytes")),
                       "us": r["us"], "calls": reps + max(3, replicas)})
        log(f"bench: {name}: {r['us']:.1f} us")
        return r

    run(DECODE_PHASES[0], wl.make_decode_case(wl.MHA_7B, dev, pa.K_AXES, pa.V_AXES,
                                              replicas=ROTATE))
    torch.cuda.empty_cache()
    gcase = wl.make_decode_case(wl.GQA, dev, pa.K_AXES, pa.V_AXES, replicas=ROTATE)
    run(DECODE_PHASES[1], gcase, ps=pa.decode_partition_for_lengths(
        gcase.lengths[:wl.GQA.num_seqs], wl.GQA.num_kv_heads, wl.GQA.block_size,
        int(max(gcase.lengths))))
    del gcase
    torch.cuda.empty_cache()
    sh8 = wl.DecodeShape("mha_7b", 64, 32, 32, 128, 16, 200_000, "fp8", wl.MHA_7B.seed)

    def dec8(out, q, k, v, t, l, maxlen, ps, ws):
        pa.pa_decode_fp8(out, q, k, v, t, l, sh8.scale, wl.FP8_SCALE, wl.FP8_SCALE, maxlen, ps,
                         ws)

    run(DECODE_PHASES[2], wl.make_decode_case(sh8, dev, pa.K_AXES, pa.V_AXES, replicas=ROTATE),
        decode=dec8)
    torch.cuda.empty_cache()
    long_case = wl.make_decode_case(wl.MIXED_DECODE, dev, pa.K_AXES, pa.V_AXES, replicas=ROTATE,
                                    num_blocks=ROTATE * 2048 + 128)
    run(DECODE_PHASES[3], long_case)
    run(DECODE_PHASES[4], long_case, ps=512)
    del long_case
    torch.cuda.empty_cache()
    # the batch's set-up kernels (cache writes, copy-on-write copies) run
    # before the next marker: the summary counts only decode kernels there
    case, alloc, _, _, samples = prefix_shared_batch(pa, wl, torch, np)
    psh = wl.PREFIX_SHARED
    groups = pa.decode_groups(case.tables, case.lengths, np.arange(len(case.lengths)) // samples,
                              psh.block_size)
    gps = pa.decode_grouped_partition(case.lengths, *groups, psh.num_q_heads, psh.num_kv_heads,
                                      psh.block_size, int(case.lengths.max()))
    r = run(DECODE_PHASES[5], case, replicas=1, ps=gps, groups=groups[:3], max_group=samples)
    phases[-1]["algorithmic_bytes"] = None  # unique bytes: see the bench row
    mark_phase(torch)
    calibrate_copy(pa, torch, np, case, alloc)
    phases.append({"phase": CAL_PHASE, "bytes_read": CALIB_PAIRS * 2 * (
        wl.PREFIX_SHARED.num_kv_heads * 16 * 128 * 2), "calls": 1})
    del case
    torch.cuda.empty_cache()
    shv = wl.MHA_7B

    def dec_valu(out, q, k, v, t, l, maxlen, ps, ws):
        pa.pa_decode(out, q, k, v, t, l, shv.scale, maxlen, ps, ws, valu=True)

    run(DECODE_PHASES[7], wl.make_decode_case(shv, dev, pa.K_AXES, pa.V_AXES, replicas=ROTATE),
        decode=dec_valu)
    with open(out_json, "w") as fh:
        json.dump({"decode_only": phases}, fh, indent=1)
    print(json.dumps({"decode_only": phases}), flush=True)


def _dispatches_by_phase(d, phases):
    """Counter rows of a rocprofv3 --pmc run, per (phase, kernel short name):
    {counter: [value per dispatch]}; phases are split at the spin-kernel
    markers in dispatch order."""
    rows = _read_counters(d)
    per_disp = {}
    for r in rows:
        key = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
        e = per_disp.setdefault(key, {"name": r.get("Kernel_Name", ""), "c": {}})
        c = r.get("Counter_Name")
        e["c"][c] = e["c"].get(c, 0.0) + float(r["Counter_Value"])
    out = {}
    phase = -1
    for key in sorted(per_disp):
        e = per_disp[key]
        if "spin_kernel" in e["name"] or "sleep" in e["name"]:
            phase += 1
            continue
        short = kernel_short_name(e["name"])
        if short is None or not 0 <= phase < len(phases):
            continue
        slot = out.setdefault((phases[phase], short), {})
        for c, v in e["c"].items():
            slot.setdefault(c, []).append(v)
    return out


def decode_counter_summary(json_file, dirs):
    """Markdown summary of rocprofv3 --pmc runs of --decode-only: per
    workload, HBM bytes per call of its decode kernels (partition kernel +
    reduce) from FETCH_SIZE / WRITE_SIZE scaled by the calibration copy's
    reading, against the algorithmic bytes; read requests by size (which
    tells whether the copy's scale carries over to the decode kernels);
    matrix-core and vector-ALU busy shares; the raw means."""
    with open(json_file) as fh:
        meta = {p["phase"]: p for p in json.load(fh)["decode_only"]}
    per = {}
    for d in dirs:
        for k, v in _dispatches_by_phase(d, DECODE_PHASES).items():
            for c, vals in v.items():
                per.setdefault(k, {})[c] = vals

    def mean(cs, c):
        v = cs.get(c)
        return sum(v) / len(v) if v else None

    cal = per.get((CAL_PHASE, "copy_blocks_kernel"), {})
    expect = meta[CAL_PHASE]["bytes_read"]
    scale = {c: expect / (mean(cal, c) * 1024) for c in ("FETCH_SIZE", "WRITE_SIZE")
             if mean(cal, c)}
    cal_req = mean(cal, "TCC_EA0_RDREQ_sum")
    bpr = expect / cal_req if cal_req else None  # bytes per counted read request
    lines = [f"Calibration: pa_copy_blocks of {CALIB_PAIRS} block pairs reads {expect} B and "
             "writes as many: " + ", ".join(f"{c} scale {v:.4f}" for c, v in scale.items())
             + (f"; {cal_req:.6g} read requests, {bpr:.2f} B per request" if bpr else ""), "",
             "| workload | HBM read B/call | HBM write B/call | algorithmic B/call | "
             "(read+write) / algorithmic |", "|---|---|---|---|---|"]
    summary = {}
    for ph in DECODE_PHASES:
        if ph == CAL_PHASE:
            continue
        rd = wr = 0.0
        have = False
        for (p2, k), cs in per.items():
            if p2 != ph or not k.startswith("decode"):
                continue
            if mean(cs, "FETCH_SIZE") is not None and "FETCH_SIZE" in scale:
                rd += mean(cs, "FETCH_SIZE") * 1024 * scale["FETCH_SIZE"]
                have = True
            if mean(cs, "WRITE_SIZE") is not None and "WRITE_SIZE" in scale:
                wr += mean(cs, "WRITE_SIZE") * 1024 * scale["WRITE_SIZE"]
        if not have:
            continue
        alg = meta[ph].get("algorithmic_bytes")
        ratio = f"{(rd + wr) / alg:.4f}" if alg else "-"
        lines.append(f"| {ph} | {rd:.5g} | {wr:.5g} | {alg if alg else 'unique bytes: bench row'}"
                     f" | {ratio} |")
        summary[ph] = {"read": rd, "write": wr, "algorithmic": alg}
    mix = []
    for (ph, k), cs in per.items():
        n = mean(cs, "TCC_EA0_RDREQ_sum")
        if not n or not (k.startswith("decode") or (k == "copy_blocks_kernel" and
                                                    ph == CAL_PHASE)):
            continue
        n32, n128 = mean(cs, "TCC_EA0_RDREQ_32B_sum") or 0, mean(cs, "TCC_BUBBLE_sum") or 0
        ndram = mean(cs, "TCC_EA0_RDREQ_DRAM_sum") or 0
        bytes_at = f"{n * bpr:.5g}" if bpr else "-"
        mix.append(f"| {ph} | {k} | {n:.6g} | {n32 / n:.4f} | {n128 / n:.4f} | "
                   f"{ndram / n:.4f} | {bytes_at} |")
    if mix:
        lines += ["", "| workload | kernel | read requests / dispatch | 32 B share | "
                  "TCC_BUBBLE (128 B) share | to-DRAM share | requests x calibration B/request |",
                  "|---|---|---|---|---|---|---|"] + mix
    busy = []
    for (ph, k), cs in per.items():
        g = mean(cs, "GRBM_GUI_ACTIVE")
        if not g or not k.startswith("decode"):
            continue
        g /= NUM_XCCS  # the csv sums the counter over the 8 XCCs
        parts = [f"{g:.4g} cycles"]
        if mean(cs, "SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            parts.append(f"matrix core busy "
                         f"{100 * mean(cs, 'SQ_VALU_MFMA_BUSY_CYCLES') / (g * NUM_SIMDS):.1f}%")
        if mean(cs, "SQ_ACTIVE_INST_VALU") is not None:
            parts.append(f"vector ALU busy "
                         f"{100 * mean(cs, 'SQ_ACTIVE_INST_VALU') / (g * NUM_CUS):.1f}%")
        busy.append(f"- {ph} / {k}: " + ", ".join(parts))
    if busy:
        lines += ["", "Busy shares (rocprof's MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x "
                  "cycles), VALUBusy = SQ_ACTIVE_INST_VALU / (CUs x cycles)):", ""] + busy
    lines += ["", "Raw means per dispatch:", "",
              "| workload | kernel | counter | mean | dispatches |", "|---|---|---|---|---|"]
    for (ph, k), cs in per.items():
        if not (k.startswith("decode") or (k == "copy_blocks_kernel" and ph == CAL_PHASE)):
            continue
        for c, vals in sorted(cs.items()):
            if c == "SQ_WAVES" and len(vals) == 0:
                continue
            lines.append(f"| {ph} | {k} | {c} | {sum(vals) / len(vals):.6g} | {len(vals)} |")
    return "\n".join(lines), summary


PHASES = ("headline decode step (7B-shaped)", "gqa decode", "prefix-shared decode + COW copy",
          "fp8 decode (7B-shaped, E4M3 K/V)", "7B-shaped decode, vector-ALU kernel and default",
          "long-context split-K decode",
          "mixed step (cache write + decode + prefill)",
          "fp8 prompt chunks (quantizing write + prefill)",
          "swap out / in (pinned host pool)", "serving loop (continuous batching)",
          "serving loop with parallel samples (grouped, then per sequence)")


def mark_phase(torch):
    """A tiny spin kernel (a few hundred cycles) that separates the workloads
    in a kernel trace; trace_summary() splits dispatches on it."""
    torch.cuda._sleep(200)


def trace_summary(d):
    """Markdown table of a rocprofv3 --kernel-trace run: libpa kernels grouped
    by workload (the spin-kernel markers), name and grid size; durations in us."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    launches = []
    phase = -1
    for r in rows:
        name = r["Kernel_Name"]
        if "spin_kernel" in name:
            phase += 1
            continue
        short = kernel_short_name(name)
        if short is None:
            continue
        label = PHASES[phase] if 0 <= phase < len(PHASES) else "-"
        wg = int(r["Workgroup_Size_X"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        launches.append((label, short, int(r["Grid_Size_X"]) // wg, wg, dur))
    # One row per (workload, kernel, grid); a kernel launched at more than
    # four grid sizes in one workload (the serving loop) gets one row.
    grids = {}
    for label, short, nwg, wg, _ in launches:
        grids.setdefault((label, short), set()).add(nwg)
    groups = {}
    for label, short, nwg, wg, dur in launches:
        many = len(grids[(label, short)]) > 4
        key = (label, short, None if many else nwg, wg)
        groups.setdefault(key, []).append(dur)
    lines = ["| workload | kernel | workgroups | threads/wg | calls | avg us | min us | max us |",
             "|---|---|---|---|---|---|---|---|"]
    for (ph, k, nwg, wg), v in groups.items():
        if nwg is None:
            g = sorted(grids[(ph, k)])
            nwg = f"{g[0]}-{g[-1]} ({len(g)} sizes)"
        lines.append(f"| {ph} | {k} | {nwg} | {wg} | {len(v)} | {sum(v) / len(v):.1f} | "
                     f"{min(v):.1f} | {max(v):.1f} |")
    return "\n".join(lines)


def kernel_short_name(name: str):
    """Readable name of a libpa kernel from a trace row, None for others.
    The tracer leaves some names mangled (a __bf16 template argument)."""
    if "pa::" in name:
        short = name.replace("(anonymous namespace)::", "").replace("void ", "")
        return short.split("(")[0].replace("pa::", "")
    m = re.match(r"_ZN2pa12_GLOBAL__N_1(\d+)", name)
    if not m:
        return None
    ident = name[m.end():m.end() + int(m.group(1))]
    rest = name[m.end() + int(m.group(1)):]
    for code, arg in (("IDF16bE", "<__bf16>"), ("IfE", "<float>"), ("ItE", "<unsigned short>")):
        if rest.startswith(code):
            return ident + arg
    return ident


# ---------------------------------------------------------------------------


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=4,
                    help="disjoint copies of the headline batch the steps rotate over")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    ap.add_argument("--rows", type=int, default=1, help="1: also measure the other rows")
    ap.add_argument("--reps", type=int, default=20, help="timed repetitions per row")
    ap.add_argument("--row-cpu-budget", type=float, default=3.0,
                    help="seconds of oracle time per row beside its GPU time (0 = skip)")
    ap.add_argument("--calibrate", action="store_true",
                    help="add one block copy of known size for the counter runs")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs into the traffic file and exit")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="print a per-kernel table of a rocprofv3 --kernel-trace run and exit")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill chunks (bf16 and fp8 caches), for counter runs")
    ap.add_argument("--prefill-counter-summary", nargs="+", metavar="PMC_DIR",
                    help="summarise rocprofv3 --pmc runs of --prefill-only and exit")
    ap.add_argument("--decode-only", metavar="OUT_JSON",
                    help="run each decode workload alone (for counter runs), write the "
                         "phases' algorithmic bytes to OUT_JSON and exit")
    ap.add_argument("--decode-counter-summary", nargs="+", metavar=("JSON", "PMC_DIR"),
                    help="summarise rocprofv3 --pmc runs of --decode-only (the JSON it wrote, "
                         "then the run directories) and exit; updates the traffic file")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary))
        return
    if args.prefill_counter_summary:
        print(prefill_counter_summary(args.prefill_counter_summary))
        return
    if args.decode_counter_summary:
        text, summary = decode_counter_summary(args.decode_counter_summary[0],
                                               args.decode_counter_summary[1:])
        print(text)
        head = summary.get(DECODE_PHASES[0])
        if head and head["read"] > 0 and head["write"] > 0:
            with open(TRAFFIC_FILE, "w") as fh:
                json.dump({"kernel": "pa_decode (decode_scan_kernel + decode_reduce_kernel)",
                           "kernel_source_sha256": kernel_source_hash(),
                           "workload": DECODE_PHASES[0],
                           "hbm_read_bytes_per_call": head["read"],
                           "hbm_write_bytes_per_call": head["write"],
                           "algorithmic_bytes_per_call": head["algorithmic"],
                           "hbm_bytes_per_launch": head["read"] + head["write"]}, fh, indent=1)
        return
    if args.pmc_summary:
        import workloads as wl
        sh = wl.MHA_7B
        block_bytes = sh.num_kv_heads * sh.block_size * sh.head_dim * 2
        s = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], block_bytes)
        print(json.dumps(s, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path "
              "shards by sequence or kv head with no exchange, and this build runs on one GPU",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_417_amd as pa
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.prefill_only:
        prefill_only(pa, wl, torch, args.reps)
        return
    if args.decode_only:
        decode_only(pa, wl, torch, np, args.reps, args.decode_only)
        return
    mark_phase(torch)
    case, h = headline(args, pa, wl, torch, np)
    K, W = args.steps, args.warmup
    src_hash = kernel_source_hash()
    result = {
        "metric": METRIC,
        "value": h["S"] / (h["ms_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": h["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q, lengths uniform [128, 4096])",
        "config": {
            "workload": "7B-shaped decode step: 64 seqs, ctx U[128,4096] (+1 per step), 32 q / "
                        "32 kv heads, head_dim 128, block 16, 200000-block pool shuffled, bf16 "
                        "KV, fp32 accumulate; cache write + decode per step",
            "global_batch": h["S"],
            "seq_len": h["seq_len"],
            "rotation": f"{h['replicas']} copies of the batch in disjoint blocks of the pool; "
                        f"step i decodes copy i mod {h['replicas']}",
            "partition_size": h["ps"],
            "parallelism": "none (1 GPU)",
        },
        "kv_gbps": h["achieved"],
        "hbm_frac": h["achieved"] / PEAK_HBM_GBPS,
        "decode_us": h["dec_avg_ms"] * 1e3,
        "roofline": {
            "kernel": "pa_decode (decode_scan_kernel + decode_reduce_kernel)",
            "bound": "hbm",
            "achieved": h["achieved"],
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": h["achieved"] / PEAK_HBM_GBPS,
            "traffic": measured_traffic(src_hash),
            "algorithmic_bytes": h["bytes_avg"],
        },
        "host_allocator_us_per_step": h["alloc_us"],
        "host_inclusive_tokens_per_s": h["host_rate"],
        "copy_reference": h["copy_ref"],
        "read_reference": h["read_ref"],
    }
    if args.cpu_budget > 0:
        log("bench: CPU baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    alloc_case = wl.DecodeCase(case.shape, case.lengths, case.perm, None, None, None, None,
                               case.k_axes, case.v_axes)
    del case
    torch.cuda.empty_cache()

    if args.rows:
        rows = {}
        log("bench: row gqa")
        mark_phase(torch)
        rows["decode_gqa"] = row_gqa(pa, wl, torch, np, args.reps, args.row_cpu_budget)
        torch.cuda.empty_cache()
        log("bench: row prefix-shared")
        mark_phase(torch)
        rows["decode_prefix_shared"], rows["copy_blocks_cow"] = row_prefix_shared(
            pa, wl, torch, np, args.reps, args.row_cpu_budget)
        torch.cuda.empty_cache()
        log("bench: row fp8 decode")
        mark_phase(torch)
        rows["decode_fp8"] = row_fp8(pa, wl, torch, np, args.reps, args.row_cpu_budget)
        torch.cuda.empty_cache()
        log("bench: row vector-ALU MHA decode")
        mark_phase(torch)
        rows["decode_mha_valu"] = row_mha_valu(pa, wl, torch, np, args.reps)
        torch.cuda.empty_cache()
        log("bench: row long-context split-K")
        mark_phase(torch)
        rows["decode_long_splitk"] = row_long(pa, wl, torch, np, args.reps, args.row_cpu_budget)
        torch.cuda.empty_cache()
        log("bench: row mixed step")
        mark_phase(torch)
        rows["prefill_chunk"], rows["cache_write"], rows["mixed_step"] = row_mixed(
            pa, wl, torch, np, args.reps, args.row_cpu_budget)
        torch.cuda.empty_cache()
        log("bench: row fp8 prefill")
        mark_phase(torch)
        rows["prefill_chunk_fp8"], rows["cache_write_fp8"] = row_fp8_prefill(
            pa, wl, torch, np, args.reps, args.row_cpu_budget)
        torch.cuda.empty_cache()
        warm_alloc = allocator_warm(pa, np, alloc_case)
        rows["allocator"] = {"host_us_per_step": h["alloc_us"],
                             "warm_binding_us_per_step": warm_alloc["binding_us"],
                             "warm_c_abi_us_per_step": warm_alloc["c_abi_us"],
                             "workload": "batch append of one token to 64 sequences + dense "
                                         "tables [64][stride] (host): host_us_per_step over the "
                                         "headline's precomputed steps; warm_*: 300 steps after "
                                         "30 untimed ones, through the binding and through the "
                                         "C ABI alone"}
        if args.row_cpu_budget > 0:
            rows["allocator"]["cpu_oracle"] = cpu_allocator_row(alloc_case, 20)
        log("bench: row prefix cache")
        rows["prefix_cache"] = row_prefix_cache(pa, wl, np, args.row_cpu_budget)
        log("bench: row swap")
        mark_phase(torch)
        rows["swap"] = row_swap(pa, wl, torch, np, args.reps, args.row_cpu_budget)
        torch.cuda.empty_cache()
        log("bench: row serving loop")
        mark_phase(torch)
        rows["serving"] = row_serving(pa, wl, torch, np, args.row_cpu_budget)
        torch.cuda.empty_cache()
        log("bench: row serving loop with parallel samples")
        mark_phase(torch)
        rows["serving_samples"] = row_serving_samples(pa, wl, torch, np)
        torch.cuda.empty_cache()
        # each HBM-bound row beside the same run's plain read stream as well
        read_gbps = h["read_ref"]["GBps"]
        for v in rows.values():
            if isinstance(v, dict) and v.get("bound") == "hbm":
                gb = v.get("GBps", v.get("GBps_unique"))
                if gb is not None:
                    v["frac_of_read_stream"] = gb / read_gbps
        result["rows"] = rows
        for k, v in rows.items():
            log(f"bench: {k}: " + ", ".join(
                f"{a}={b:.4g}" if isinstance(b, float) else
                (f"{a}={b['value']:.4g} {b['unit']}" if isinstance(b, dict) and "value" in b
                 else f"{a}={b}")
                for a, b in v.items() if a != "workload"))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Decode-step benchmark of the paged-KV attention path on one MI355X.

One step = one decode iteration of the whole batch through the C ABI:
  host allocator appends one token per sequence (slots, on-demand blocks) ->
  block tables / lengths / slots copied to the device ->
  pa_cache_write of the new tokens' K/V -> pa_decode (partition + split-K
  reduce kernels).
Workload (7B-shaped batch): 64 sequences with context lengths uniform in
[128, 4096], 32 query heads = 32 kv heads, head_dim 128, block_size 16,
blocks shuffled across a 200,000-block pool, bf16 K/V, fp32 accumulation.
Inputs are synthetic (seeded N(0,1)), resident in HBM before timing starts.

Prints one JSON line.  `value` = decoded tokens per second (sequences per
step / step time).  `roofline` covers pa_decode (both of its kernels), timed
with HIP events on the launch stream inside the timed region; `cpu_baseline`
is the fp64 oracle on a bounded sample of the same batch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode tokens/s and achieved KV HBM GB/s (% of MI355X peak), 1 GPU"
PEAK_HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_mha_7b_traffic.json")
KERNEL_SOURCES = ("decode_mfma.hip", "decode_reduce.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_417_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def algorithmic_bytes(lengths, hq, hkv, d, bs, e_kv=2, e_q=2):
    """K/V bytes of valid tokens + q + fp32 output + block-table entries + lengths."""
    kv = sum(int(L) for L in lengths) * hkv * d * 2 * e_kv
    s = len(lengths)
    tables = sum(-(-int(L) // bs) for L in lengths) * 4
    return kv + s * hq * d * e_q + s * hq * d * 4 + tables + s * 4


def measured_traffic(src_hash: str, n_launch_bytes: float):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on this exact kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle, single-threaded, on whole sequences of the batch until
    the time budget is spent (at least one)."""
    import numpy as np
    import torch

    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paged_helpers import gather_blocks, host_bits

    sh = case.shape
    order = list(range(len(case.lengths)))
    done, elapsed, tokens = 0, 0.0, 0
    for s in order:
        k_sub, v_sub, t_sub, l_sub = gather_blocks(case.k_pool, case.v_pool, case.tables,
                                                   case.lengths, [s], sh.block_size)
        q_sub = host_bits(case.q[s:s + 1])
        t0 = time.perf_counter()
        oracle.decode(q_sub, k_sub, v_sub, t_sub, l_sub, sh.scale, case.k_axes, case.v_axes)
        elapsed += time.perf_counter() - t0
        done += 1
        tokens += int(l_sub[0])
        if elapsed >= budget_s:
            break
    return {"value": done / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {len(order)} sequences of the batch ({tokens} context tokens), "
                      f"all {sh.num_q_heads} heads, fp64, one thread, {elapsed:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the CPU baseline (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or kv head with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_417_amd as pa
    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    sh = wl.MHA_7B
    K, W = args.steps, args.warmup
    log(f"bench: building {sh.name} batch (S={sh.num_seqs}, NB={sh.num_blocks})")
    case = wl.make_decode_case(sh, dev, pa.K_AXES, pa.V_AXES, extra_table_slots=K + W + 1)
    S = sh.num_seqs
    stride = case.tables.shape[1]
    pad = sh.num_blocks - 1

    # The allocator replays the prompts: with free_order = the batch's
    # permutation it hands out exactly the blocks the batch was laid into.
    alloc = pa.Allocator(sh.num_blocks, sh.block_size, free_order=case.perm)
    ids = np.arange(S, dtype=np.int64)
    for s in ids:
        alloc.create(int(s))
    alloc.batch_append(ids, case.lengths)
    t_chk, l_chk = alloc.batch_tables(ids, stride, pad)
    assert (t_chk == case.tables).all() and (l_chk == case.lengths).all()

    gen = wl.make_generator(sh.seed + 1000, dev)
    nsteps = K + W
    k_new = wl.randn((nsteps, S, sh.num_kv_heads, sh.head_dim), torch.bfloat16, gen, dev)
    v_new = wl.randn((nsteps, S, sh.num_kv_heads, sh.head_dim), torch.bfloat16, gen, dev)
    q_all = wl.randn((nsteps, S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    out = torch.empty((S, sh.num_q_heads, sh.head_dim), device=dev)
    max_len = int(case.lengths.max()) + nsteps
    ps = args.partition_size
    ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                             max_len, ps, dev)
    ps_used = ps or pa.pa_decode_default_partition(S, sh.num_kv_heads, sh.block_size, max_len)

    # double-buffered pinned host staging and device copies
    h_slots = [torch.zeros(S, dtype=torch.int64).pin_memory() for _ in range(2)]
    h_tabs = [torch.zeros((S, stride), dtype=torch.int32).pin_memory() for _ in range(2)]
    h_lens = [torch.zeros(S, dtype=torch.int32).pin_memory() for _ in range(2)]
    d_slots = [torch.zeros(S, dtype=torch.int64, device=dev) for _ in range(2)]
    d_tabs = [torch.zeros((S, stride), dtype=torch.int32, device=dev) for _ in range(2)]
    d_lens = [torch.zeros(S, dtype=torch.int32, device=dev) for _ in range(2)]
    copied = [None, None]
    ones = np.ones(S, dtype=np.int32)
    stream = torch.cuda.current_stream()
    dec_events = []
    step_lengths = []

    def step(i, timed):
        b = i % 2
        if copied[b] is not None:
            copied[b].synchronize()  # staging buffer b free again
        slots_np = h_slots[b].numpy()
        alloc.batch_append(ids, ones, slots_out=slots_np)
        tabs_np, lens_np = h_tabs[b].numpy(), h_lens[b].numpy()
        alloc.batch_tables(ids, stride, pad, tables_out=tabs_np, lens_out=lens_np)
        d_slots[b].copy_(h_slots[b], non_blocking=True)
        d_tabs[b].copy_(h_tabs[b], non_blocking=True)
        d_lens[b].copy_(h_lens[b], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        copied[b] = ev
        pa.pa_cache_write(k_new[i], v_new[i], case.k_pool, case.v_pool, d_slots[b])
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        pa.pa_decode(out, q_all[i], case.k_pool, case.v_pool, d_tabs[b], d_lens[b], sh.scale,
                     max_len, ps, ws)
        if timed:
            e1.record(stream)
            dec_events.append((e0, e1))
            step_lengths.append(lens_np.copy())

    log(f"bench: warmup {W} steps, partition {ps_used}")
    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    log(f"bench: timing {K} steps")
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i, True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    dec_ms = [a.elapsed_time(b) for a, b in dec_events]
    dec_avg_ms = sum(dec_ms) / len(dec_ms)
    bytes_avg = sum(algorithmic_bytes(L, sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                                      sh.block_size) for L in step_lengths) / len(step_lengths)
    achieved = bytes_avg / (dec_avg_ms * 1e-3) / 1e9
    assert torch.isfinite(out).all()
    log(f"bench: step {ms_step:.3f} ms, decode {dec_avg_ms * 1e3:.1f} us "
        f"(min {min(dec_ms) * 1e3:.1f}, max {max(dec_ms) * 1e3:.1f}), "
        f"{achieved:.0f} GB/s algorithmic")

    src_hash = kernel_source_hash()
    traffic = measured_traffic(src_hash, bytes_avg)
    result = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) K/V/q, lengths uniform [128, 4096])",
        "config": {
            "workload": "mha_7b decode step: 64 seqs, ctx U[128,4096] (+1 per step), 32 q / "
                        "32 kv heads, head_dim 128, block 16, 200000-block pool, bf16 KV, "
                        "fp32 accumulate",
            "global_batch": S,
            "seq_len": int(np.mean(step_lengths[-1])),
            "partition_size": ps_used,
            "parallelism": "none (1 GPU)",
        },
        "kv_gbps": achieved,
        "hbm_frac": achieved / PEAK_HBM_GBPS,
        "decode_us": dec_avg_ms * 1e3,
        "roofline": {
            "kernel": "pa_decode (decode_mfma_kernel + decode_reduce_kernel)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes": bytes_avg,
        },
    }
    if args.cpu_budget > 0:
        log("bench: CPU baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

"""Test plumbing shared by the GPU parity tests: moving device pools and
tables to the host in the form the oracle takes.  No attention arithmetic
here; the oracle does that."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Device or host tensor -> numpy array of its stored bits (fp32 as
    float32, bf16 as uint16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.uint8:  # E4M3 codes
        return t.numpy()
    raise TypeError(t.dtype)


def gather_blocks(k_pool, v_pool, tables, lengths, rows, block_size):
    """Copy the blocks that sequences ``rows`` use to the host.

    Returns (k_sub, v_sub, sub_tables, sub_lengths) where the sub pools hold
    only those blocks (same axis order as the device pools) and sub_tables
    index into them."""
    tables = np.asarray(tables)
    ids, remap = [], {}
    sub_tables = np.zeros((len(rows), tables.shape[1]), dtype=np.int32)
    for i, s in enumerate(rows):
        n = -(-int(lengths[s]) // block_size)
        for j in range(n):
            b = int(tables[s][j])
            if b not in remap:
                remap[b] = len(ids)
                ids.append(b)
            sub_tables[i, j] = remap[b]
    if not ids:
        ids = [0]
    idx = torch.as_tensor(ids, device=k_pool.device, dtype=torch.long)
    k_sub = host_bits(k_pool.index_select(0, idx))
    v_sub = host_bits(v_pool.index_select(0, idx))
    return k_sub, v_sub, sub_tables, np.asarray([lengths[s] for s in rows], dtype=np.int32)


def oracle_decode_rows(q, k_pool, v_pool, tables, lengths, rows, block_size, scale,
                       k_axes, v_axes, k_scale=1.0, v_scale=1.0):
    """fp64 oracle outputs for sequences ``rows`` of a device batch (pools of
    fp32, bf16 or E4M3 codes with their scales)."""
    k_sub, v_sub, t_sub, l_sub = gather_blocks(k_pool, v_pool, tables, lengths, rows, block_size)
    q_sub = host_bits(q[torch.as_tensor(list(rows), device=q.device, dtype=torch.long)])
    return oracle.decode(q_sub, k_sub, v_sub, t_sub, l_sub, scale, k_axes, v_axes,
                         k_scale, v_scale)


def chunked_checksum(t: torch.Tensor, chunk: int = 1 << 28) -> tuple[int, int]:
    """Two position-sensitive int64 checksums of a tensor's bytes, computed on
    its device in chunks (for pools too large to copy)."""
    w = t.view(-1).view(torch.int32) if t.element_size() * t.numel() % 4 == 0 else None
    assert w is not None
    s1 = torch.zeros((), dtype=torch.int64, device=t.device)
    s2 = torch.zeros((), dtype=torch.int64, device=t.device)
    for lo in range(0, w.numel(), chunk):
        part = w[lo:lo + chunk].to(torch.int64)
        pos = torch.arange(lo, lo + part.numel(), device=t.device, dtype=torch.int64) % 1000003
        s1 += part.sum()
        s2 += (part * (pos + 1)).sum()
    return int(s1), int(s2)


def oracle_threads() -> int:
    """Host threads for the oracle runs of the full-size parity tests: the
    cores this process may use, at most 16 (one GPU's share of a host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _run_threaded(fn, tasks, weights):
    """fn over tasks on oracle_threads() threads, heaviest first (the C
    oracle runs outside Python's lock).  Results come back in task order."""
    from concurrent.futures import ThreadPoolExecutor
    oracle._load()  # load the library before the threads start
    order = sorted(range(len(tasks)), key=lambda i: -weights[i])
    out = [None] * len(tasks)
    with ThreadPoolExecutor(oracle_threads()) as ex:
        futs = {i: ex.submit(fn, tasks[i]) for i in order}
        for i, f in futs.items():
            out[i] = f.result()
    return out


def oracle_decode_all(q, k_pool, v_pool, tables, lengths, block_size, scale, k_axes, v_axes,
                      k_scale=1.0, v_scale=1.0, rows=None):
    """fp64 oracle outputs [len(rows)][Hq][D] for every sequence of a device
    batch (or for ``rows``): the used blocks are copied to the host once and
    each sequence is one task on the host threads."""
    rows = list(range(len(lengths))) if rows is None else list(rows)
    if not rows:
        return np.zeros((0,) + tuple(q.shape[1:]), np.float64)
    k_sub, v_sub, t_sub, l_sub = gather_blocks(k_pool, v_pool, tables, lengths, rows, block_size)
    q_sub = host_bits(q[torch.as_tensor(rows, device=q.device, dtype=torch.long)])

    def one(i):
        return oracle.decode(q_sub[i:i + 1], k_sub, v_sub, t_sub[i:i + 1], l_sub[i:i + 1], scale,
                             k_axes, v_axes, k_scale, v_scale)[0]

    return np.stack(_run_threaded(one, list(range(len(rows))), [int(x) for x in l_sub]))


def oracle_prefill_all(q, k_pool, v_pool, tables, cu_q_lens, context_lens, block_size, scale,
                       k_axes, v_axes, k_scale=1.0, v_scale=1.0, rows_per_task=32):
    """fp64 oracle outputs [Tq][Hq][D] of a whole prefill batch.  Each task is
    a slice of one request's rows i0..i1-1, posed to the oracle as a request
    of its own: i1 - i0 new rows over ctx - qlen + i1 keys, so its rows sit
    at the same absolute positions and see the same keys.  Rows of requests
    whose chunk is longer than their context are left at zero."""
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    ctx = np.asarray(context_lens, dtype=np.int64)
    R = len(ctx)
    k_sub, v_sub, t_sub, _ = gather_blocks(k_pool, v_pool, tables, ctx, range(R), block_size)
    q_host = host_bits(q)
    out = np.zeros(tuple(q.shape), np.float64)
    tasks = []
    for r in range(R):
        qlen = int(cu[r + 1] - cu[r])
        if qlen > ctx[r]:
            continue
        for i0 in range(0, qlen, rows_per_task):
            tasks.append((r, i0, min(qlen, i0 + rows_per_task)))

    def one(t):
        r, i0, i1 = t
        q0 = int(cu[r])
        keys = int(ctx[r]) - int(cu[r + 1] - cu[r]) + i1
        out[q0 + i0:q0 + i1] = oracle.prefill(
            q_host[q0 + i0:q0 + i1], k_sub, v_sub, t_sub[r:r + 1],
            np.array([0, i1 - i0], np.int32), np.array([keys], np.int32), scale, k_axes, v_axes,
            k_scale, v_scale)

    _run_threaded(one, tasks, [(t[2] - t[1]) * (int(ctx[t[0]]) + t[2]) for t in tasks])
    return out

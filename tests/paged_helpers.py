"""Test plumbing shared by the GPU parity tests: moving device pools and
tables to the host in the form the oracle takes.  No attention arithmetic
here; the oracle does that."""
from __future__ import annotations

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

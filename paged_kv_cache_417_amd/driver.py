"""Continuous-batching serving loop over the C ABI (argument marshalling only).

``ServingLoop`` owns the device K/V pools, an optional pinned host pool for
swap space, the allocator and the scheduler.  Each ``step()`` asks the C++
scheduler for a plan and carries it out on the GPU, in the order the plan
requires: swap-out copies, swap-in copies, copy-on-write copies, the cache
write of the step's new positions, the prompt chunks (pa_prefill_chunk) and
the decode batch (pa_decode).  There is no model: the caller supplies the K/V
rows of every new position and the q rows of every query (``rows_fn``,
``q_fn``, each called once per batch with a list of (sequence id, positions)
and returning the rows of all entries back to back), so the loop exercises
the whole library end to end on synthetic data.

Parallel sampling (《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1: the samples drawn
from one prompt share its KV blocks): a request added with sample ids is
forked by the scheduler once its prompt is written, and its samples decode
side by side.  A decode batch holding such runs goes through
pa_decode_grouped, each request's run one group (pa_decode_groups derives the
blocks its members share), so the shared prompt blocks are read once per
group, at the partition size pa_decode_grouped_partition picks for the batch
and with the streaming load policy (no block is read twice).  The result is
pa_decode's up to the merge's rounding (bit for bit where the shared region
ends on a partition boundary).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (Allocator, Scheduler, decode_grouped_partition, decode_groups, decode_workspace,
               kv_cache_shapes,
               pa_cache_write, pa_cache_write_fp8, pa_copy_blocks, pa_decode, pa_decode_fp8,
               pa_decode_grouped, pa_decode_grouped_fp8, pa_prefill_chunk, pa_prefill_chunk_fp8,
               pa_swap_blocks)


class _Staging:
    """A step's small integer arrays (slots, tables, lengths, prefix sums,
    group arrays, block pairs) go to the device together: they are packed
    into one pinned buffer and sent with one asynchronous copy, instead of
    one synchronous upload from pageable memory each.  Two buffers alternate;
    a buffer is refilled only once its previous copy has completed, and its
    device twin is overwritten only by a later copy on the same stream, after
    the kernels that read it."""

    def __init__(self, device, nbytes=1 << 20):
        self.dev = device
        self.i = 0
        self.host = [None, None]
        self.devbuf = [None, None]
        self.done = [None, None]
        self.cap = [0, 0]
        self.want = nbytes

    def begin(self):
        b = self.i
        if self.done[b] is not None:
            self.done[b].synchronize()
        self.parts = []
        self.off = 0

    def put(self, arr):
        """Queue a numpy array; returns its index for ``send``'s list."""
        arr = np.ascontiguousarray(arr)
        self.parts.append((self.off, arr))
        self.off += -(-arr.nbytes // 16) * 16  # keep every part 16-byte aligned
        return len(self.parts) - 1

    def send(self):
        """One host-to-device copy of everything queued; device tensors in
        ``put`` order, each with its array's dtype and shape."""
        b = self.i
        self.i ^= 1
        need = max(self.off, 16)
        if self.cap[b] < need:
            self.cap[b] = max(need, self.want, 2 * self.cap[b])
            self.host[b] = torch.empty(self.cap[b], dtype=torch.uint8, pin_memory=True)
            self.devbuf[b] = torch.empty(self.cap[b], dtype=torch.uint8, device=self.dev)
        hb = self.host[b].numpy()
        for off, arr in self.parts:
            hb[off:off + arr.nbytes] = arr.view(np.uint8).reshape(-1)
        self.devbuf[b][:self.off].copy_(self.host[b][:self.off], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(torch.cuda.current_stream())
        self.done[b] = ev
        out = []
        for off, arr in self.parts:
            t = self.devbuf[b][off:off + arr.nbytes].view(_TORCH_OF[arr.dtype.str[1:]])
            out.append(t.view(arr.shape))
        return out


_TORCH_OF = {"i4": torch.int32, "i8": torch.int64}


class ServingLoop:
    def __init__(self, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                 max_num_seqs, max_batched_tokens, max_prefill_chunk, max_context_len,
                 host_blocks=0, free_order=None, device="cuda", dtype=torch.bfloat16,
                 fp8_scales=None, group_samples=True):
        """fp8_scales=(k_scale, v_scale): keep the cache as OCP E4M3 codes
        (uint8 pools) and use the fp8 calls; new rows are still bf16.
        group_samples=False decodes sample runs one sequence at a time
        (pa_decode with the cache-keeping policy) instead of grouped."""
        self.group_samples = group_samples
        self.time_decode = False  # True: event-time every decode call (decode_ms())
        self._dec_events = []
        self.bs, self.hq, self.hkv, self.d = block_size, num_q_heads, num_kv_heads, head_dim
        self.max_ctx = int(max_context_len)
        self.dev, self.dtype = device, dtype
        self.fp8 = fp8_scales
        pool_dtype = torch.uint8 if fp8_scales else dtype
        fill = 0x7F if fp8_scales else float("nan")
        kshape, vshape = kv_cache_shapes(num_blocks, num_kv_heads, block_size, head_dim)
        self.k = torch.full(kshape, fill, dtype=pool_dtype, device=device)
        self.v = torch.full(vshape, fill, dtype=pool_dtype, device=device)
        self.alloc = Allocator(num_blocks, block_size, free_order=free_order)
        self.hk = self.hv = None
        if host_blocks:
            self.alloc.set_swap_space(host_blocks)
            hk, hv = kv_cache_shapes(host_blocks, num_kv_heads, block_size, head_dim)
            self.hk = torch.empty(hk, dtype=pool_dtype, pin_memory=True)
            self.hv = torch.empty(hv, dtype=pool_dtype, pin_memory=True)
        self.sched = Scheduler(self.alloc, max_num_seqs, max_batched_tokens, max_prefill_chunk)
        self.stride = -(-self.max_ctx // block_size) + 1
        self.pad = num_blocks - 1
        # sized for pa_decode_grouped, which needs more than pa_decode
        self.ws = decode_workspace(max_num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                   self.max_ctx, 0, device, grouped=True)
        self.scale = head_dim ** -0.5
        self.request_of = {}  # sample sequence id -> its request id
        self.staging = _Staging(device)
        self.grouped_steps = 0       # decode steps that ran grouped
        self.shared_block_reads = 0  # group-shared blocks, summed over those steps

    def add(self, rid, n_prompt, max_new, tokens=None, samples=()):
        """Queue a request; samples: sequence ids of its parallel samples
        2..n."""
        if n_prompt + max_new > self.max_ctx:
            raise ValueError("request longer than max_context_len")
        self.sched.add(rid, n_prompt, max_new, tokens, samples=samples)
        for x in samples:
            self.request_of[int(x)] = rid

    def decode_grouping(self, seq_ids):
        """seq_group for pa_decode_groups: each run of two or more sequences
        of one request (the scheduler keeps them adjacent) is a group, every
        other sequence -1; None when there is no group."""
        n = len(seq_ids)
        ro = self.request_of
        owner = np.fromiter((ro.get(x, x) for x in seq_ids), dtype=np.int64, count=n)
        if n < 2:
            return None
        # runs of equal owners: start index and length of each
        starts = np.flatnonzero(np.concatenate(([True], owner[1:] != owner[:-1])))
        lengths = np.diff(np.append(starts, n))
        multi = lengths > 1
        if not multi.any():
            return None
        seq_group = np.full(n, -1, dtype=np.int32)
        run_group = np.cumsum(multi) - 1  # group id of each multi-member run
        member = np.repeat(multi, lengths)
        seq_group[member] = np.repeat(run_group[multi], lengths[multi]).astype(np.int32)
        return seq_group

    def step(self, rows_fn, q_fn):
        """One scheduler step on the GPU.  rows_fn(entries) -> (k, v)
        [total][Hkv][D]; q_fn(entries) -> q [total][Hq][D], entries being
        [(request id, positions)].  Returns (plan, decode output or None,
        prefill output or None, finished ids)."""
        dev = self.dev
        p = self.sched.step()
        # every integer array of the step goes up in one pinned copy
        st = self.staging
        st.begin()
        i_out = st.put(np.asarray(p["swap_out"], np.int32)) if len(p["swap_out"]) else None
        i_in = st.put(np.asarray(p["swap_in"], np.int32)) if len(p["swap_in"]) else None
        i_cow = st.put(np.asarray(p["cow"], np.int32)) if len(p["cow"]) else None
        # new positions: decode positions first, then each chunk's
        dpos = np.fromiter((ctx - 1 for _, ctx in p["decode"]), dtype=np.int64,
                           count=len(p["decode"]))
        dec_entries = [(x[0], dpos[i:i + 1]) for i, x in enumerate(p["decode"])]
        pre_entries = [(rid, np.arange(start, start + n)) for rid, start, n in p["prefill"]]
        i_slots = st.put(np.asarray(p["slots"], np.int64)) if dec_entries or pre_entries else None
        if p["prefill"]:
            ids = [x[0] for x in p["prefill"]]
            t, _ = self.alloc.batch_tables(ids, self.stride, self.pad)
            qlens = np.array([x[2] for x in p["prefill"]], dtype=np.int32)
            # the chunk's context ends at its last new position
            ctx = np.array([x[1] + x[2] for x in p["prefill"]], dtype=np.int32)
            cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
            i_pre = (st.put(t), st.put(cu), st.put(ctx))
        groups = None
        if p["decode"]:
            ids = [x[0] for x in p["decode"]]
            t, lens = self.alloc.batch_tables(ids, self.stride, self.pad)
            seq_group = self.decode_grouping(ids)
            if seq_group is not None and self.group_samples:
                off, sg, shared, largest = decode_groups(t, lens, seq_group, self.bs)
                gps = decode_grouped_partition(lens, off, sg, shared, largest, self.hq,
                                               self.hkv, self.bs, self.max_ctx)
                groups = (st.put(off), st.put(sg), st.put(shared), largest, gps)
                self.grouped_steps += 1
                self.shared_block_reads += int(shared.sum())
            i_dec = (st.put(t), st.put(lens))
        d = st.send()
        if i_out is not None:
            pa_swap_blocks(self.k, self.v, self.hk, self.hv, d[i_out])
        if i_in is not None:
            pa_swap_blocks(self.hk, self.hv, self.k, self.v, d[i_in])
        if i_cow is not None:
            pa_copy_blocks(self.k, self.v, d[i_cow])
        if i_slots is not None:
            k, v = rows_fn(dec_entries + pre_entries)
            if self.fp8:
                pa_cache_write_fp8(k, v, self.k, self.v, d[i_slots], *self.fp8)
            else:
                pa_cache_write(k, v, self.k, self.v, d[i_slots])
        pre_out = dec_out = None
        if p["prefill"]:
            pre_out = torch.empty((int(cu[-1]), self.hq, self.d), device=dev)
            args = (d[i_pre[0]], d[i_pre[1]], d[i_pre[2]], self.scale)
            if self.fp8:
                pa_prefill_chunk_fp8(pre_out, q_fn(pre_entries), self.k, self.v, *args, *self.fp8,
                                     int(qlens.max()), self.max_ctx)
            else:
                pa_prefill_chunk(pre_out, q_fn(pre_entries), self.k, self.v, *args,
                                 int(qlens.max()), self.max_ctx)
        if p["decode"]:
            q = q_fn(dec_entries)
            dec_out = torch.empty((len(ids), self.hq, self.d), device=dev)
            t, lens = d[i_dec[0]], d[i_dec[1]]
            if groups:
                gps = groups[4]
                groups = (d[groups[0]], d[groups[1]], d[groups[2]], groups[3])
            if self.time_decode:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ev[0].record()
            if groups and self.fp8:
                pa_decode_grouped_fp8(dec_out, q, self.k, self.v, t, lens, self.scale, *self.fp8,
                                      self.max_ctx, *groups, gps, self.ws)
            elif groups:
                pa_decode_grouped(dec_out, q, self.k, self.v, t, lens, self.scale, self.max_ctx,
                                  *groups, gps, self.ws)
            elif self.fp8:
                pa_decode_fp8(dec_out, q, self.k, self.v, t, lens, self.scale, *self.fp8,
                              self.max_ctx, 0, self.ws, kv_reuse=seq_group is not None)
            else:
                pa_decode(dec_out, q, self.k, self.v, t, lens, self.scale, self.max_ctx, 0,
                          self.ws, kv_reuse=seq_group is not None)
            if self.time_decode:
                ev[1].record()
                self._dec_events.append(ev)
        fin = self.sched.complete()
        return p, dec_out, pre_out, fin

    def decode_ms(self):
        """Total event time of the decode calls timed so far (synchronizes)."""
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in self._dec_events)

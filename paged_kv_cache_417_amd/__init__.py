"""Python binding of libpa (paged-KV attention for MI355X / gfx950).

A thin ctypes layer: every function here marshals torch tensors into the raw
pointers and sizes of the C ABI declared in ``include/pa.h`` and raises
:class:`PAError` on a non-OK status.  All computation happens in the HIP
kernels of ``libpa.so``; if the library is missing, importing this package
fails.  PyTorch provides device memory and the current stream only.

Storage layout (the ABI): ``k_cache [NB][Hkv][BS][D]``, ``v_cache
[NB][Hkv][D][BS]``; see :func:`kv_cache_shapes`.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")
# Host-sanitizer runs only: PA_HOST_LIB names a CPU-only build of the
# library's host code (allocator, scheduler, group derivation, error text)
# made with -fsanitize=address,undefined.  Only the symbols it exports are
# declared; the device calls are absent from it (using one raises
# AttributeError), so nothing runs in place of a kernel.
_HOST_LIB = os.environ.get("PA_HOST_LIB")

PA_OK = 0
PA_ERR_INVALID_ARG = 1
PA_ERR_OUT_OF_BLOCKS = 2
PA_ERR_NOT_FOUND = 3
PA_ERR_UNSUPPORTED = 4
PA_ERR_DEVICE = 5
PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1
PA_DTYPE_FP8_E4M3 = 2  # OCP E4M3 codes, stored in torch.uint8 tensors
PA_DECODE_KV_REUSE = 1
PA_DECODE_VALU = 2  # bf16: the vector-ALU decode kernel instead of the matrix-core one
PA_DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20  # the device scratch behind pa_decode_noalloc

# Axis order of the two pools, in the letters b (block), h (kv head),
# r (row = token within block), d (head dim).
K_AXES = "bhrd"
V_AXES = "bhdr"

# Every symbol the header declares; the CPU tests check the library exports them.
EXPORTED = (
    "pa_last_error", "pa_cache_write", "pa_copy_blocks", "pa_read_stream", "pa_decode_default_partition",
    "pa_decode_workspace_size", "pa_decode", "pa_decode_ex", "pa_prefill_chunk",
    "pa_allocator_create",
    "pa_allocator_destroy", "pa_seq_create", "pa_seq_fork", "pa_seq_append", "pa_seq_free",
    "pa_seq_length", "pa_seq_block_table", "pa_allocator_stats", "pa_block_refcount",
    "pa_batch_append", "pa_batch_tables", "pa_seq_create_prefix", "pa_seq_append_tokens",
    "pa_batch_append_tokens", "pa_prefix_cache_stats", "pa_allocator_set_swap_space",
    "pa_seq_swap_out", "pa_seq_swap_in", "pa_seq_is_swapped", "pa_swap_stats", "pa_swap_blocks",
    "pa_cache_write_fp8", "pa_decode_fp8", "pa_prefill_chunk_fp8", "pa_seq_blocks_needed", "pa_seq_num_blocks",
    "pa_sched_create", "pa_sched_destroy", "pa_sched_add", "pa_sched_step", "pa_sched_complete",
    "pa_sched_stats", "pa_decode_grouped", "pa_decode_grouped_fp8", "pa_decode_groups",
    "pa_decode_grouped_workspace_size", "pa_decode_grouped_partition",
    "pa_decode_partition_for_lengths", "pa_decode_noalloc", "pa_seq_create_prefix_ex", "pa_prefix_cache_offload",
    "pa_prefix_host_stats", "pa_sched_add_samples",
)


class PAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libpa status {status}: {message}")
        self.status = status


class OutOfBlocks(PAError):
    pass


class AllocatorStats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_free", ctypes.c_int32),
                ("num_used", ctypes.c_int32), ("num_shared", ctypes.c_int32),
                ("cow_copies", ctypes.c_int64)]


class SwapStats(ctypes.Structure):
    _fields_ = [("num_host_blocks", ctypes.c_int32), ("num_host_free", ctypes.c_int32),
                ("swapped_seqs", ctypes.c_int32), ("swap_out_blocks", ctypes.c_int64),
                ("swap_in_blocks", ctypes.c_int64)]


class SchedPlan(ctypes.Structure):
    _P64, _P32 = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)
    _fields_ = [("decode_ids", _P64), ("decode_lens", _P32), ("prefill_ids", _P64),
                ("prefill_starts", _P32), ("prefill_lens", _P32), ("preempted_ids", _P64),
                ("cap_seqs", ctypes.c_int32), ("slots", _P64), ("cap_slots", ctypes.c_int32),
                ("cow_pairs", _P32), ("cap_cow", ctypes.c_int32), ("swap_out_pairs", _P32),
                ("swap_in_pairs", _P32), ("cap_swap_pairs", ctypes.c_int32),
                ("n_decode", ctypes.c_int32), ("n_prefill", ctypes.c_int32),
                ("n_preempted", ctypes.c_int32), ("n_slots", ctypes.c_int32),
                ("n_cow", ctypes.c_int32), ("n_swap_out", ctypes.c_int32),
                ("n_swap_in", ctypes.c_int32)]


class SchedStats(ctypes.Structure):
    _fields_ = [("waiting", ctypes.c_int32), ("running", ctypes.c_int32),
                ("swapped", ctypes.c_int32), ("running_seqs", ctypes.c_int32),
                ("finished", ctypes.c_int64), ("swap_preemptions", ctypes.c_int64),
                ("recompute_preemptions", ctypes.c_int64), ("forked_samples", ctypes.c_int64)]


class PrefixHostStats(ctypes.Structure):
    _fields_ = [("host_cached_blocks", ctypes.c_int32), ("offloaded_blocks", ctypes.c_int64),
                ("reloaded_blocks", ctypes.c_int64)]


class PrefixStats(ctypes.Structure):
    _fields_ = [("queried_blocks", ctypes.c_int64), ("hit_blocks", ctypes.c_int64),
                ("cached_blocks", ctypes.c_int32), ("cached_free_blocks", ctypes.c_int32)]


def _declare(lib):
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    st = ctypes.c_int
    # host arrays travel as plain addresses (numpy's .ctypes.data): a typed
    # pointer cast costs microseconds per argument on every call
    pi32 = pi64 = ctypes.c_void_p
    sig = {
        "pa_last_error": (ctypes.c_char_p, []),
        "pa_cache_write": (st, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]),
        "pa_copy_blocks": (st, [vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]),
        "pa_read_stream": (st, [vp, ctypes.c_size_t, vp, vp]),
        "pa_decode_default_partition": (i32, [i32, i32, i32, i32]),
        "pa_decode_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "pa_decode_grouped_workspace_size": (sz, [i32, i32, i32, i32, i32, i32, i32]),
        "pa_decode": (st, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                           i32, vp, sz, ctypes.c_int, vp]),
        "pa_decode_ex": (st, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32, i32,
                              i32, vp, sz, ctypes.c_int, ctypes.c_uint32, vp]),
        "pa_prefill_chunk": (st, [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                  i32, i32, i32, f32, ctypes.c_int, vp]),
        "pa_allocator_create": (st, [i32, i32, pi32, ctypes.POINTER(vp)]),
        "pa_allocator_destroy": (None, [vp]),
        "pa_seq_create": (st, [vp, i64]),
        "pa_seq_fork": (st, [vp, i64, i64]),
        "pa_seq_append": (st, [vp, i64, i32, pi64, pi32, i32, pi32]),
        "pa_seq_free": (st, [vp, i64]),
        "pa_seq_length": (st, [vp, i64, pi32]),
        "pa_seq_block_table": (st, [vp, i64, pi32, i32, pi32]),
        "pa_allocator_stats": (st, [vp, ctypes.POINTER(AllocatorStats)]),
        "pa_block_refcount": (st, [vp, i32, pi32]),
        "pa_batch_append": (st, [vp, i32, pi64, pi32, pi64, pi32, i32, pi32]),
        "pa_batch_tables": (st, [vp, i32, pi64, pi32, i32, i32, pi32]),
        "pa_seq_create_prefix": (st, [vp, i64, pi32, i32, i32, pi32]),
        "pa_seq_append_tokens": (st, [vp, i64, pi32, i32, pi64, pi32, i32, pi32]),
        "pa_batch_append_tokens": (st, [vp, i32, pi64, pi32, pi32, pi64, pi32, i32, pi32]),
        "pa_prefix_cache_stats": (st, [vp, ctypes.POINTER(PrefixStats)]),
        "pa_seq_create_prefix_ex": (st, [vp, i64, pi32, i32, i32, pi32, pi32, i32, pi32]),
        "pa_prefix_cache_offload": (st, [vp, i32, pi32, i32, pi32]),
        "pa_prefix_host_stats": (st, [vp, ctypes.POINTER(PrefixHostStats)]),
        "pa_allocator_set_swap_space": (st, [vp, i32]),
        "pa_seq_swap_out": (st, [vp, i64, pi32, i32, pi32]),
        "pa_seq_swap_in": (st, [vp, i64, pi32, i32, pi32]),
        "pa_seq_is_swapped": (st, [vp, i64, pi32]),
        "pa_swap_stats": (st, [vp, ctypes.POINTER(SwapStats)]),
        "pa_swap_blocks": (st, [vp, vp, i32, vp, vp, i32, vp, i32, i32, i32, i32, ctypes.c_int,
                                vp]),
        "pa_seq_blocks_needed": (st, [vp, i64, i32, pi32]),
        "pa_seq_num_blocks": (st, [vp, i64, pi32]),
        "pa_sched_create": (st, [vp, i32, i32, i32, ctypes.POINTER(vp)]),
        "pa_sched_destroy": (None, [vp]),
        "pa_sched_add": (st, [vp, i64, i32, i32, pi32]),
        "pa_sched_add_samples": (st, [vp, i64, i32, i32, pi32, pi64, i32]),
        "pa_sched_step": (st, [vp, ctypes.POINTER(SchedPlan)]),
        "pa_sched_complete": (st, [vp, pi64, i32, pi32]),
        "pa_sched_stats": (st, [vp, ctypes.POINTER(SchedStats)]),
        "pa_prefill_chunk_fp8": (st, [vp, vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                      i32, i32, i32, i32, f32, f32, f32, vp]),
        "pa_cache_write_fp8": (st, [vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                    f32, vp]),
        "pa_decode_fp8": (st, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32, f32,
                               f32, i32, i32, vp, sz, ctypes.c_uint32, vp]),
        "pa_decode_grouped": (st, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32, f32,
                                   i32, i32, vp, vp, vp, i32, i32, vp, sz, ctypes.c_int,
                                   ctypes.c_uint32, vp]),
        "pa_decode_noalloc": (st, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                   f32, i32, i32, ctypes.c_int, ctypes.c_uint32, vp]),
        "pa_decode_groups": (st, [pi32, i32, pi32, pi32, i32, i32, i32, pi32, pi32, pi32]),
        "pa_decode_grouped_partition": (i32, [pi32, pi32, pi32, pi32, i32, i32, i32, i32, i32,
                                              i32, i32]),
        "pa_decode_partition_for_lengths": (i32, [pi32, i32, i32, i32, i32]),
        "pa_decode_grouped_fp8": (st, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                       f32, f32, f32, i32, i32, vp, vp, vp, i32, i32, vp, sz,
                                       ctypes.c_uint32, vp]),
    }
    for name, (res, args) in sig.items():
        if _HOST_LIB and not hasattr(lib, name):
            continue
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


if _HOST_LIB:
    _lib = ctypes.CDLL(_HOST_LIB)
else:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python paged_kv_cache_417_amd/build.py` (hipcc, gfx950)")
    _lib = ctypes.CDLL(LIB_PATH)
_declare(_lib)


def lib():
    return _lib


def _check(status: int):
    if status != PA_OK:
        msg = _lib.pa_last_error().decode(errors="replace")
        if status == PA_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(status, msg)
        raise PAError(status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PA_DTYPE_BF16
    if t.dtype == torch.float32:
        return PA_DTYPE_F32
    if t.dtype == torch.uint8:
        return PA_DTYPE_FP8_E4M3
    return 99  # rejected by the library as an invalid dtype


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def kv_cache_shapes(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int):
    """Shapes of (k_cache, v_cache) in the library's layout."""
    return ((num_blocks, num_kv_heads, block_size, head_dim),
            (num_blocks, num_kv_heads, head_dim, block_size))


def _geometry(k_cache: torch.Tensor):
    nb, hkv, bs, d = k_cache.shape
    return nb, hkv, bs, d


# ---------------------------------------------------------------------------
# device calls


def pa_cache_write(k_new, v_new, k_cache, v_cache, slot_mapping, stream=None) -> None:
    nb, hkv, bs, d = _geometry(k_cache)
    _check(_lib.pa_cache_write(_p(k_new), _p(v_new), _p(k_cache), _p(v_cache), _p(slot_mapping),
                               k_new.shape[0], hkv, d, bs, nb, _dtype_code(k_cache),
                               ctypes.c_void_p(_stream(stream))))


def pa_copy_blocks(k_cache, v_cache, src_dst, stream=None) -> None:
    nb, hkv, bs, d = _geometry(k_cache)
    n = src_dst.numel() // 2
    _check(_lib.pa_copy_blocks(_p(k_cache), _p(v_cache), _p(src_dst), n, hkv, d, bs, nb,
                               _dtype_code(k_cache), ctypes.c_void_p(_stream(stream))))


READ_STREAM_SINK_WORDS = 32768


def pa_read_stream(src, sink, stream=None) -> None:
    """Read every byte of the device tensor ``src`` once (the plain streaming
    read the decode rates are compared with); ``sink`` is a device int32 or
    uint32 tensor of READ_STREAM_SINK_WORDS words that receives one XOR fold
    per workgroup."""
    if sink.numel() * sink.element_size() < 4 * READ_STREAM_SINK_WORDS:
        raise PAError(PA_ERR_INVALID_ARG, "pa_read_stream: sink smaller than 8192 words")
    _check(_lib.pa_read_stream(_p(src), src.numel() * src.element_size(), _p(sink),
                               ctypes.c_void_p(_stream(stream))))


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, src_dst, stream=None) -> None:
    """Copy whole blocks src_dst[i][0] of (src_k, src_v) to src_dst[i][1] of
    (dst_k, dst_v): one pool on the device, the other a pinned host pool of the
    same block layout (``torch.empty(..., pin_memory=True)``).  src_dst must
    live on the device or in pinned host memory."""
    nb_s, hkv, bs, d = _geometry(src_k)
    nb_d, hkv2, bs2, d2 = _geometry(dst_k)
    if (hkv, bs, d) != (hkv2, bs2, d2) or src_k.dtype != dst_k.dtype:
        raise PAError(PA_ERR_INVALID_ARG, "pa_swap_blocks: pools differ in geometry or dtype")
    n = src_dst.numel() // 2
    _check(_lib.pa_swap_blocks(_p(src_k), _p(src_v), nb_s, _p(dst_k), _p(dst_v), nb_d,
                               _p(src_dst), n, hkv, d, bs, _dtype_code(src_k),
                               ctypes.c_void_p(_stream(stream))))


def pa_decode_default_partition(num_seqs, num_kv_heads, block_size, max_context_len) -> int:
    return int(_lib.pa_decode_default_partition(num_seqs, num_kv_heads, block_size,
                                                max_context_len))


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_context_len, partition_size=0) -> int:
    n = _lib.pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_context_len, partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(PA_ERR_INVALID_ARG, "pa_decode_workspace_size: invalid sizes")
    return int(n)


def decode_partition_for_lengths(lens, num_kv_heads, block_size, max_context_len) -> int:
    """pa_decode_partition_for_lengths on a host array of context lengths:
    the partition size for pa_decode of this batch."""
    import numpy as np
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    ps = _lib.pa_decode_partition_for_lengths(_i32p(lens), len(lens), num_kv_heads, block_size,
                                              int(max_context_len))
    if ps <= 0:
        raise PAError(PA_ERR_INVALID_ARG, _lib.pa_last_error().decode(errors="replace"))
    return int(ps)


def pa_decode_grouped_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                     max_context_len, partition_size=0) -> int:
    n = _lib.pa_decode_grouped_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              block_size, max_context_len, partition_size)
    if n == ctypes.c_size_t(-1).value:
        raise PAError(PA_ERR_INVALID_ARG, "pa_decode_grouped_workspace_size: invalid sizes")
    return int(n)


def decode_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                     partition_size=0, device="cuda", grouped=False):
    """A device buffer large enough for the split-K partials of pa_decode
    (grouped: of pa_decode_grouped, which needs more), or None."""
    size = pa_decode_grouped_workspace_size if grouped else pa_decode_workspace_size
    n = size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
             partition_size)
    return None if n == 0 else torch.empty(n, dtype=torch.uint8, device=device)


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
              partition_size=0, workspace=None, stream=None, kv_reuse=False,
              valu=False) -> None:
    """Paged decode; kv_reuse=True (pa_decode_ex with PA_DECODE_KV_REUSE) for
    batches whose sequences share blocks; valu=True (PA_DECODE_VALU) runs a
    bf16 batch on the vector-ALU kernel."""
    nb, hkv, bs, d = _geometry(k_cache)
    s, hq, _ = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), block_tables.shape[1],
            _p(context_lens), s, hq, hkv, d, bs, nb, float(scale), int(max_context_len),
            int(partition_size), _p(workspace), ws_bytes, _dtype_code(k_cache))
    flags = (PA_DECODE_KV_REUSE if kv_reuse else 0) | (PA_DECODE_VALU if valu else 0)
    if flags:
        _check(_lib.pa_decode_ex(*args, flags, ctypes.c_void_p(_stream(stream))))
    else:
        _check(_lib.pa_decode(*args, ctypes.c_void_p(_stream(stream))))


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, partition_size=0, stream=None, kv_reuse=False) -> None:
    """pa_decode without a workspace: the split-K partials use the scratch
    the library keeps on the device (for callers that cannot allocate)."""
    nb, hkv, bs, d = _geometry(k_cache)
    s, hq, _ = q.shape
    _check(_lib.pa_decode_noalloc(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                  block_tables.shape[1], _p(context_lens), s, hq, hkv, d, bs, nb,
                                  float(scale), int(max_context_len), int(partition_size),
                                  _dtype_code(k_cache), PA_DECODE_KV_REUSE if kv_reuse else 0,
                                  ctypes.c_void_p(_stream(stream))))


def pa_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, group_offsets, seq_group, group_shared, max_group_size,
                      partition_size=0, workspace=None, stream=None, kv_reuse=False) -> None:
    """Paged decode with groups of sequences that share leading blocks: each
    group's shared region is read once (int32 device tensors: group_offsets
    [G+1], seq_group [S], group_shared [G]).  decode_grouped_partition gives
    the partition size for such a batch, decode_workspace(..., grouped=True)
    a workspace large enough."""
    nb, hkv, bs, d = _geometry(k_cache)
    s, hq, _ = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode_grouped(
        _p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), block_tables.shape[1],
        _p(context_lens), s, hq, hkv, d, bs, nb, float(scale), int(max_context_len),
        int(partition_size), _p(group_offsets), _p(seq_group), _p(group_shared),
        group_shared.numel(), int(max_group_size), _p(workspace), ws_bytes,
        _dtype_code(k_cache), PA_DECODE_KV_REUSE if kv_reuse else 0,
        ctypes.c_void_p(_stream(stream))))


def decode_groups(tables, lens, seq_group, block_size):
    """Group arrays for pa_decode_grouped (pa_decode_groups on host arrays).
    seq_group [S] gives each sequence's group id, or -1; ids run 0..G-1 in
    sequence order and each group's members are consecutive.  Returns int32
    numpy arrays (group_offsets [G+1], seq_group [S], group_shared [G]) and
    the largest group size; group_shared counts the leading blocks every
    member holds equal to the first member.  Raises ValueError for a
    malformed grouping."""
    import numpy as np
    seq_group = np.ascontiguousarray(seq_group, dtype=np.int32)
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    S = len(seq_group)
    G = int(seq_group.max()) + 1 if S else 0
    offsets = np.zeros(G + 1, np.int32)
    shared = np.zeros(max(G, 1), np.int32)
    largest = ctypes.c_int32(0)
    st = _lib.pa_decode_groups(_i32p(tables), tables.shape[1] if tables.ndim == 2 else 1,
                               _i32p(lens), _i32p(seq_group), S, int(block_size), G,
                               _i32p(offsets), _i32p(shared), ctypes.byref(largest))
    if st == PA_ERR_INVALID_ARG:
        raise ValueError(_lib.pa_last_error().decode(errors="replace"))
    _check(st)
    return offsets, seq_group, shared[:G], largest.value


def decode_grouped_partition(lens, group_offsets, seq_group, group_shared, max_group_size,
                             num_q_heads, num_kv_heads, block_size, max_context_len) -> int:
    """pa_decode_grouped_partition on host arrays (those decode_groups
    returns): the partition size for a grouped decode of this batch."""
    import numpy as np
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    offsets = np.ascontiguousarray(group_offsets, dtype=np.int32)
    seq_group = np.ascontiguousarray(seq_group, dtype=np.int32)
    shared = np.ascontiguousarray(group_shared, dtype=np.int32)
    ps = _lib.pa_decode_grouped_partition(_i32p(lens), _i32p(offsets), _i32p(seq_group),
                                          _i32p(shared), len(lens), len(shared),
                                          int(max_group_size), num_q_heads, num_kv_heads,
                                          block_size, int(max_context_len))
    if ps <= 0:
        raise PAError(PA_ERR_INVALID_ARG, _lib.pa_last_error().decode(errors="replace"))
    return int(ps)


def pa_decode_grouped_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale,
                          v_scale, max_context_len, group_offsets, seq_group, group_shared,
                          max_group_size, partition_size=0, workspace=None, stream=None,
                          kv_reuse=False) -> None:
    """pa_decode_grouped over uint8 (E4M3) caches; q is bf16."""
    nb, hkv, bs, d = _geometry(k_cache)
    s, hq, _ = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode_grouped_fp8(
        _p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables), block_tables.shape[1],
        _p(context_lens), s, hq, hkv, d, bs, nb, float(scale), float(k_scale), float(v_scale),
        int(max_context_len), int(partition_size), _p(group_offsets), _p(seq_group),
        _p(group_shared), group_shared.numel(), int(max_group_size), _p(workspace), ws_bytes,
        PA_DECODE_KV_REUSE if kv_reuse else 0, ctypes.c_void_p(_stream(stream))))


def pa_cache_write_fp8(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale, v_scale,
                       stream=None) -> None:
    """Quantizing write of bf16/fp32 rows into uint8 (E4M3) caches."""
    nb, hkv, bs, d = _geometry(k_cache)
    _check(_lib.pa_cache_write_fp8(_p(k_new), _p(v_new), _dtype_code(k_new), _p(k_cache),
                                   _p(v_cache), _p(slot_mapping), k_new.shape[0], hkv, d, bs, nb,
                                   float(k_scale), float(v_scale),
                                   ctypes.c_void_p(_stream(stream))))


def pa_decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
                  max_context_len, partition_size=0, workspace=None, stream=None,
                  kv_reuse=False) -> None:
    """Paged decode over uint8 (E4M3) caches; q is bf16."""
    nb, hkv, bs, d = _geometry(k_cache)
    s, hq, _ = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_decode_fp8(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                              block_tables.shape[1], _p(context_lens), s, hq, hkv, d, bs, nb,
                              float(scale), float(k_scale), float(v_scale), int(max_context_len),
                              int(partition_size), _p(workspace), ws_bytes,
                              PA_DECODE_KV_REUSE if kv_reuse else 0,
                              ctypes.c_void_p(_stream(stream))))


def pa_prefill_chunk_fp8(out, q, k_cache, v_cache, block_tables, cu_q_lens, context_lens, scale,
                         k_scale, v_scale, max_q_len, max_context_len, stream=None) -> None:
    """Chunked causal prefill over uint8 (E4M3) caches; q is bf16."""
    nb, hkv, bs, d = _geometry(k_cache)
    tq, hq, _ = q.shape
    _check(_lib.pa_prefill_chunk_fp8(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                     block_tables.shape[1], _p(cu_q_lens), _p(context_lens),
                                     context_lens.shape[0], tq, int(max_q_len),
                                     int(max_context_len), hq, hkv, d, bs, nb, float(scale),
                                     float(k_scale), float(v_scale),
                                     ctypes.c_void_p(_stream(stream))))


def pa_prefill_chunk(out, q, k_cache, v_cache, block_tables, cu_q_lens, context_lens, scale,
                     max_q_len, max_context_len, stream=None) -> None:
    nb, hkv, bs, d = _geometry(k_cache)
    tq, hq, _ = q.shape
    _check(_lib.pa_prefill_chunk(_p(out), _p(q), _p(k_cache), _p(v_cache), _p(block_tables),
                                 block_tables.shape[1], _p(cu_q_lens), _p(context_lens),
                                 context_lens.shape[0], tq, int(max_q_len), int(max_context_len),
                                 hq, hkv, d, bs, nb, float(scale), _dtype_code(k_cache),
                                 ctypes.c_void_p(_stream(stream))))


# ---------------------------------------------------------------------------
# host allocator


def _i64p(a):
    """Address of a C-contiguous int64 numpy array (for a c_void_p argument)."""
    return a.ctypes.data


def _i32p(a):
    """Address of a C-contiguous int32 numpy array (for a c_void_p argument)."""
    return a.ctypes.data


class Allocator:
    """Owner of one ``pa_allocator`` handle (host memory only)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        import numpy as np
        self._np = np
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.num_host_blocks = 0
        h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            self._free_order = np.ascontiguousarray(free_order, dtype=np.int32)
            fo = _i32p(self._free_order)
        _check(_lib.pa_allocator_create(self.num_blocks, self.block_size, fo, ctypes.byref(h)))
        self._h = h
        self._pairs_buf = np.zeros((1, 2), dtype=np.int32)
        self._ncow = ctypes.c_int32(0)
        self._ncow_ref = ctypes.byref(self._ncow)

    def close(self):
        if getattr(self, "_h", None) and _lib is not None:  # _lib is None at interpreter exit
            _lib.pa_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def create(self, seq_id: int):
        _check(_lib.pa_seq_create(self._h, seq_id))

    def fork(self, parent: int, child: int):
        _check(_lib.pa_seq_fork(self._h, parent, child))

    def append(self, seq_id: int, n_tokens: int):
        """Returns (slots int64 [n], cow_pairs int32 [k][2])."""
        np = self._np
        slots = np.zeros(max(n_tokens, 1), dtype=np.int64)
        pairs = np.zeros((1, 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_lib.pa_seq_append(self._h, seq_id, n_tokens, _i64p(slots), _i32p(pairs), 1,
                                  ctypes.byref(ncow)))
        return slots[:n_tokens], pairs[:ncow.value]

    def batch_append(self, seq_ids, n_tokens, slots_out=None, pairs_out=None):
        """Append n_tokens[i] to seq_ids[i] for all i at once (all or nothing).
        Returns (slots, cow_pairs)."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        nt = np.ascontiguousarray(n_tokens, dtype=np.int32)
        total = int(nt.sum())
        slots = slots_out if slots_out is not None else np.zeros(max(total, 1), dtype=np.int64)
        if pairs_out is not None:
            pairs = pairs_out
        else:  # a buffer kept across calls; the pairs returned are a copy
            if self._pairs_buf.shape[0] < len(ids):
                self._pairs_buf = np.zeros((len(ids), 2), dtype=np.int32)
            pairs = self._pairs_buf
        ncow = self._ncow
        _check(_lib.pa_batch_append(self._h, len(ids), ids.ctypes.data, nt.ctypes.data,
                                    slots.ctypes.data, pairs.ctypes.data, pairs.shape[0],
                                    self._ncow_ref))
        n = ncow.value
        return slots[:total], (pairs[:n] if pairs_out is not None else pairs[:n].copy())

    def create_prefix(self, seq_id: int, tokens, max_cached_tokens=None) -> int:
        """New sequence reusing the cached blocks of the prompt ``tokens``;
        returns the positions covered (its length)."""
        np = self._np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        mc = len(t) if max_cached_tokens is None else int(max_cached_tokens)
        n = ctypes.c_int32(0)
        _check(_lib.pa_seq_create_prefix(self._h, seq_id, _i32p(t) if len(t) else None, len(t),
                                         mc, ctypes.byref(n)))
        return n.value

    def create_prefix_ex(self, seq_id: int, tokens, max_cached_tokens=None):
        """create_prefix that also brings the prompt's host-tier hits back;
        returns (positions covered, pairs int32 [k][2] (host block, device
        block) to copy host -> device before decoding)."""
        np = self._np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        mc = len(t) if max_cached_tokens is None else int(max_cached_tokens)
        cap = max(len(t) // self.block_size, 1)
        pairs = np.zeros((cap, 2), dtype=np.int32)
        n, k = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(_lib.pa_seq_create_prefix_ex(self._h, seq_id, t.ctypes.data if len(t) else None,
                                            len(t), mc, ctypes.byref(n), pairs.ctypes.data,
                                            cap, ctypes.byref(k)))
        return n.value, pairs[:k.value].copy()

    def offload(self, max_blocks: int):
        """Move up to max_blocks of the oldest released prefix-cache blocks
        to the host tier; returns pairs int32 [k][2] (device block, host
        block) to copy device -> host before the device pool is written."""
        np = self._np
        cap = max(int(max_blocks), 1)
        pairs = np.zeros((cap, 2), dtype=np.int32)
        k = ctypes.c_int32(0)
        _check(_lib.pa_prefix_cache_offload(self._h, int(max_blocks), pairs.ctypes.data, cap,
                                            ctypes.byref(k)))
        return pairs[:k.value].copy()

    def host_stats(self) -> dict:
        st = PrefixHostStats()
        _check(_lib.pa_prefix_host_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in PrefixHostStats._fields_}

    def append_tokens(self, seq_id: int, tokens):
        """Append positions with their token ids (full blocks get registered).
        Returns (slots, cow_pairs)."""
        np = self._np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.zeros(max(len(t), 1), dtype=np.int64)
        pairs = np.zeros((1, 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_lib.pa_seq_append_tokens(self._h, seq_id, _i32p(t) if len(t) else None, len(t),
                                         _i64p(slots), _i32p(pairs), 1, ctypes.byref(ncow)))
        return slots[:len(t)], pairs[:ncow.value]

    def batch_append_tokens(self, seq_ids, tokens_per_seq):
        """``tokens_per_seq[i]`` is appended to ``seq_ids[i]``, all at once."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        nt = np.array([len(t) for t in tokens_per_seq], dtype=np.int32)
        flat = np.ascontiguousarray(np.concatenate([np.asarray(t, dtype=np.int32)
                                                    for t in tokens_per_seq] or
                                                   [np.zeros(0, np.int32)]), dtype=np.int32)
        flat = flat if len(flat) else np.zeros(1, dtype=np.int32)
        total = int(nt.sum())
        slots = np.zeros(max(total, 1), dtype=np.int64)
        pairs = np.zeros((max(len(ids), 1), 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_lib.pa_batch_append_tokens(self._h, len(ids), _i64p(ids), _i32p(nt),
                                           _i32p(flat), _i64p(slots), _i32p(pairs),
                                           pairs.shape[0], ctypes.byref(ncow)))
        return slots[:total], pairs[:ncow.value]

    def set_swap_space(self, num_host_blocks: int):
        _check(_lib.pa_allocator_set_swap_space(self._h, num_host_blocks))
        self.num_host_blocks = int(num_host_blocks)

    def _swap(self, fn, seq_id):
        np = self._np
        cap = len(self.block_table(seq_id)) or 1
        pairs = np.zeros((cap, 2), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(fn(self._h, seq_id, _i32p(pairs), cap, ctypes.byref(n)))
        return pairs[:n.value]

    def swap_out(self, seq_id: int):
        """Returns pairs [n][2] (device block, host block) to copy out."""
        return self._swap(_lib.pa_seq_swap_out, seq_id)

    def swap_in(self, seq_id: int):
        """Returns pairs [n][2] (host block, device block) to copy in."""
        return self._swap(_lib.pa_seq_swap_in, seq_id)

    def is_swapped(self, seq_id: int) -> bool:
        r = ctypes.c_int32(0)
        _check(_lib.pa_seq_is_swapped(self._h, seq_id, ctypes.byref(r)))
        return bool(r.value)

    def swap_stats(self) -> dict:
        st = SwapStats()
        _check(_lib.pa_swap_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in SwapStats._fields_}

    def prefix_stats(self) -> dict:
        st = PrefixStats()
        _check(_lib.pa_prefix_cache_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in PrefixStats._fields_}

    def batch_tables(self, seq_ids, stride: int, pad_value: int = 0, tables_out=None,
                     lens_out=None):
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = tables_out if tables_out is not None else np.zeros((len(ids), stride), np.int32)
        lens = lens_out if lens_out is not None else np.zeros(len(ids), np.int32)
        _check(_lib.pa_batch_tables(self._h, len(ids), ids.ctypes.data, tables.ctypes.data,
                                    stride, pad_value, lens.ctypes.data))
        return tables, lens

    def free(self, seq_id: int):
        _check(_lib.pa_seq_free(self._h, seq_id))

    def length(self, seq_id: int) -> int:
        n = ctypes.c_int32(0)
        _check(_lib.pa_seq_length(self._h, seq_id, ctypes.byref(n)))
        return n.value

    def block_table(self, seq_id: int):
        np = self._np
        n = ctypes.c_int32(0)
        cap = self.length(seq_id) // self.block_size + 2
        out = np.zeros(cap, dtype=np.int32)
        _check(_lib.pa_seq_block_table(self._h, seq_id, _i32p(out), cap, ctypes.byref(n)))
        return out[:n.value]

    def stats(self) -> dict:
        st = AllocatorStats()
        _check(_lib.pa_allocator_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in AllocatorStats._fields_}

    def refcount(self, block: int) -> int:
        r = ctypes.c_int32(0)
        _check(_lib.pa_block_refcount(self._h, block, ctypes.byref(r)))
        return r.value


class Scheduler:
    """Owner of one ``pa_sched`` (continuous batching over an Allocator)."""

    def __init__(self, alloc: "Allocator", max_num_seqs: int, max_batched_tokens: int,
                 max_prefill_chunk: int):
        import numpy as np
        self._np = np
        self.alloc = alloc  # keeps the allocator alive
        self.max_num_seqs = int(max_num_seqs)
        self.max_batched_tokens = int(max_batched_tokens)
        h = ctypes.c_void_p()
        _check(_lib.pa_sched_create(alloc._h, self.max_num_seqs, self.max_batched_tokens,
                                    int(max_prefill_chunk), ctypes.byref(h)))
        self._h = h
        n, t, nb = self.max_num_seqs, self.max_batched_tokens, alloc.num_blocks
        self._a = {"decode_ids": np.zeros(n, np.int64), "decode_lens": np.zeros(n, np.int32),
                   "prefill_ids": np.zeros(n, np.int64), "prefill_starts": np.zeros(n, np.int32),
                   "prefill_lens": np.zeros(n, np.int32), "preempted_ids": np.zeros(n, np.int64),
                   "slots": np.zeros(t, np.int64), "cow_pairs": np.zeros((n, 2), np.int32),
                   "swap_out_pairs": np.zeros((nb, 2), np.int32),
                   "swap_in_pairs": np.zeros((nb, 2), np.int32)}
        self._plan = SchedPlan()
        for k, v in self._a.items():
            ptype = ctypes.c_int64 if v.dtype == np.int64 else ctypes.c_int32
            setattr(self._plan, k, v.ctypes.data_as(ctypes.POINTER(ptype)))
        self._plan.cap_seqs, self._plan.cap_slots, self._plan.cap_cow = n, t, n
        self._swap_cap(max(nb, alloc.num_host_blocks))
        self._fin = np.zeros(n, np.int64)

    def _swap_cap(self, cap):
        """(Re)size the swap pair arrays: a step needs room for the larger of
        the device and host pool sizes."""
        np = self._np
        for k in ("swap_out_pairs", "swap_in_pairs"):
            self._a[k] = np.zeros((cap, 2), np.int32)
            setattr(self._plan, k, self._a[k].ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        self._plan.cap_swap_pairs = cap

    def close(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pa_sched_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, rid: int, n_prompt: int, max_new: int, tokens=None, samples=()):
        """Queue a request; samples lists the sequence ids of its parallel
        samples 2..n (pa_sched_add_samples), none for one sample."""
        np = self._np
        t = None
        if tokens is not None:
            self._tok = np.ascontiguousarray(tokens, dtype=np.int32)
            t = _i32p(self._tok)
        ids = np.ascontiguousarray(list(samples), dtype=np.int64)
        _check(_lib.pa_sched_add_samples(self._h, rid, n_prompt, max_new, t,
                                         _i64p(ids) if len(ids) else None, 1 + len(ids)))

    def step(self) -> dict:
        """Plan one step; returns copies of the filled plan arrays."""
        if self._plan.cap_swap_pairs < self.alloc.num_host_blocks:
            self._swap_cap(self.alloc.num_host_blocks)
        _check(_lib.pa_sched_step(self._h, ctypes.byref(self._plan)))
        p, a = self._plan, self._a
        return {"decode": list(zip(a["decode_ids"][:p.n_decode].tolist(),
                                   a["decode_lens"][:p.n_decode].tolist())),
                "prefill": list(zip(a["prefill_ids"][:p.n_prefill].tolist(),
                                    a["prefill_starts"][:p.n_prefill].tolist(),
                                    a["prefill_lens"][:p.n_prefill].tolist())),
                "preempted": a["preempted_ids"][:p.n_preempted].tolist(),
                "slots": a["slots"][:p.n_slots].copy(),
                "cow": a["cow_pairs"][:p.n_cow].copy(),
                "swap_out": a["swap_out_pairs"][:p.n_swap_out].copy(),
                "swap_in": a["swap_in_pairs"][:p.n_swap_in].copy()}

    def complete(self) -> list:
        n = ctypes.c_int32(0)
        _check(_lib.pa_sched_complete(self._h, _i64p(self._fin), len(self._fin),
                                      ctypes.byref(n)))
        return self._fin[:n.value].tolist()

    def stats(self) -> dict:
        st = SchedStats()
        _check(_lib.pa_sched_stats(self._h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in SchedStats._fields_}

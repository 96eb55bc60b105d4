"""fp64 CPU oracle for paged-KV attention (ctypes wrapper over ``liboracle.so``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the product library: it has its own C source (``oracle.c``), its own
loader, and takes storage layouts as axis strings so that it does not depend on
how the product arranges K and V inside a block.

Sources (page title, section) cited in the functions below:
  [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》
  [VF] 《大模型推理：vLLM大模型推理框架（附下载）》
  [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》
  [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》

Arrays are numpy.  bf16 data is passed as its raw 16-bit patterns
(``numpy.uint16``); fp32 as ``numpy.float32``.  Pools are 4-D arrays whose axes
are named by a 4-letter string over {b: block, h: kv head, r: row in block,
d: head dim}; e.g. ``"bhrd"`` for ``[NB][Hkv][BS][D]``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at a deliberately broken build of oracle.c to
# show that the pins catch it; nothing else sets this.
_OVERRIDE = os.environ.get("PA_ORACLE_LIB")
_lib = None

F32 = 0
BF16 = 1
FP8 = 2  # OCP E4M3 codes stored as uint8


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (plain -O2, IEEE semantics, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Strides(ctypes.Structure):
    _fields_ = [("block", ctypes.c_int64), ("head", ctypes.c_int64),
                ("row", ctypes.c_int64), ("dim", ctypes.c_int64)]


def _load():
    global _lib
    if _lib is None:
        path = _OVERRIDE or _LIB_PATH
        if not _OVERRIDE and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.orc_widen.restype = dbl
        lib.orc_widen.argtypes = [vp, i64, ctypes.c_int]
        lib.orc_decode.restype = None
        lib.orc_decode.argtypes = [vp, vp, ctypes.c_int, vp, _Strides, vp, _Strides,
                                   ctypes.c_int, vp, i32, vp, i32, i32, i32, i32, i32, dbl, dbl,
                                   dbl]
        lib.orc_e4m3_decode.restype = dbl
        lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        lib.orc_cache_write_fp8.restype = None
        lib.orc_cache_write_fp8.argtypes = [vp, vp, ctypes.c_int, vp, _Strides, vp, _Strides, vp,
                                            i32, i32, i32, i32, ctypes.c_float, ctypes.c_float]
        lib.orc_prefill.restype = None
        lib.orc_prefill.argtypes = [vp, vp, ctypes.c_int, vp, _Strides, vp, _Strides,
                                    ctypes.c_int, vp, i32, vp, vp, i32, i32, i32, i32, i32, dbl,
                                    dbl, dbl]
        lib.orc_cache_write.restype = None
        lib.orc_cache_write.argtypes = [vp, vp, vp, _Strides, vp, _Strides, vp, i32, i32, i32,
                                        i32, i32]
        lib.orc_copy_blocks.restype = None
        lib.orc_copy_blocks.argtypes = [vp, _Strides, vp, _Strides, vp, i32, i32, i32, i32, i32]
        lib.orc_swap_blocks.restype = None
        lib.orc_swap_blocks.argtypes = [vp, _Strides, vp, _Strides, vp, _Strides, vp, _Strides,
                                        vp, i32, i32, i32, i32, i32]
        lib.orc_unpage.restype = None
        lib.orc_unpage.argtypes = [vp, _Strides, ctypes.c_int, vp, i32, i32, i32, i32, vp]
        _lib = lib
    return _lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    raise TypeError(f"oracle takes float32, bf16 bits (uint16) or E4M3 codes (uint8), "
                    f"got {a.dtype}")


def _strides(pool: np.ndarray, axes: str) -> _Strides:
    if pool.ndim != 4 or sorted(axes) != sorted("bhrd"):
        raise ValueError("pool must be 4-D with axes a permutation of 'bhrd'")
    el = pool.itemsize
    st = {ax: pool.strides[i] // el for i, ax in enumerate(axes)}
    return _Strides(st["b"], st["h"], st["r"], st["d"])


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    a = np.asarray(a) if dtype is None else np.asarray(a, dtype=dtype)
    return np.ascontiguousarray(a)


def pool_dims(pool: np.ndarray, axes: str):
    """(num_blocks, num_kv_heads, block_size, head_dim) of a pool."""
    n = {ax: pool.shape[i] for i, ax in enumerate(axes)}
    return n["b"], n["h"], n["r"], n["d"]


def widen(a: np.ndarray) -> np.ndarray:
    """Stored elements (fp32, or bf16 bits) as float64, exactly."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise TypeError(a.dtype)


def unpage(pool: np.ndarray, axes: str, table, length: int, head: int) -> np.ndarray:
    """K (or V) rows 0..length-1 of one kv head of one sequence, as [L][D] float64."""
    lib = _load()
    _, _, bs, d = pool_dims(pool, axes)
    table = _c(table, np.int32)
    out = np.zeros((max(length, 0), d), dtype=np.float64)
    lib.orc_unpage(_ptr(pool), _strides(pool, axes), _dtype_code(pool), _ptr(table),
                   bs, length, head, d, _ptr(out))
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale,
           k_axes="bhrd", v_axes="bhrd", k_scale=1.0, v_scale=1.0) -> np.ndarray:
    """Paged decode attention, fp64 ([VE] §3.1 and §3.3).

    q: [S][Hq][D] (fp32 or bf16 bits); pools: 4-D with the given axes (fp32,
    bf16 bits, or E4M3 codes whose values are multiplied by k_scale / v_scale);
    block_tables: [S][stride] int32; context_lens: [S] int32.
    Returns out[S][Hq][D] float64.
    """
    lib = _load()
    q = _c(q)
    block_tables = _c(block_tables, np.int32)
    context_lens = _c(context_lens, np.int32)
    s, hq, d = q.shape
    _, hkv, bs, dk = pool_dims(k_cache, k_axes)
    assert dk == d and hq % hkv == 0
    assert k_cache.dtype == v_cache.dtype
    out = np.zeros((s, hq, d), dtype=np.float64)
    lib.orc_decode(_ptr(out), _ptr(q), _dtype_code(q),
                   _ptr(k_cache), _strides(k_cache, k_axes),
                   _ptr(v_cache), _strides(v_cache, v_axes), _dtype_code(k_cache),
                   _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                   s, hq, hkv, d, bs, float(scale), float(k_scale), float(v_scale))
    return out


def e4m3_decode(codes) -> np.ndarray:
    """Values of OCP E4M3 codes (uint8), float64."""
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.orc_e4m3_decode(int(x)) for x in c.reshape(-1)]).reshape(c.shape)


def e4m3_encode(x) -> np.ndarray:
    """Nearest OCP E4M3 codes of float32 values (ties to even, saturating)."""
    lib = _load()
    a = np.asarray(x, dtype=np.float32)
    return np.array([lib.orc_e4m3_encode(float(v)) for v in a.reshape(-1)],
                    dtype=np.uint8).reshape(a.shape)


def cache_write_fp8(k_new, v_new, k_cache, v_cache, slot_mapping, k_scale, v_scale,
                    k_axes="bhrd", v_axes="bhrd") -> None:
    """Quantizing cache write into uint8 E4M3 pools: code = nearest E4M3 of
    (x / scale) computed in binary32."""
    lib = _load()
    k_new, v_new = _c(k_new), _c(v_new)
    slots = _c(slot_mapping, np.int64)
    t, hkv, d = k_new.shape
    _, hk2, bs, d2 = pool_dims(k_cache, k_axes)
    assert (hk2, d2) == (hkv, d) and k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
    lib.orc_cache_write_fp8(_ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(k_cache),
                            _strides(k_cache, k_axes), _ptr(v_cache), _strides(v_cache, v_axes),
                            _ptr(slots), t, hkv, d, bs, float(k_scale), float(v_scale))


def prefill(q, k_cache, v_cache, block_tables, cu_q_lens, context_lens, scale,
            k_axes="bhrd", v_axes="bhrd", k_scale=1.0, v_scale=1.0) -> np.ndarray:
    """Paged causal prefill of query chunks, fp64 ([VI] §1, mixed phases).

    q: [Tq][Hq][D]; cu_q_lens: [R+1] prefix sums of new rows per request;
    context_lens: [R] keys per request including the chunk's own.
    Returns out[Tq][Hq][D] float64.
    """
    lib = _load()
    q = _c(q)
    block_tables = _c(block_tables, np.int32)
    cu_q_lens = _c(cu_q_lens, np.int32)
    context_lens = _c(context_lens, np.int32)
    tq, hq, d = q.shape
    _, hkv, bs, _ = pool_dims(k_cache, k_axes)
    r = context_lens.shape[0]
    out = np.zeros((tq, hq, d), dtype=np.float64)
    lib.orc_prefill(_ptr(out), _ptr(q), _dtype_code(q),
                    _ptr(k_cache), _strides(k_cache, k_axes),
                    _ptr(v_cache), _strides(v_cache, v_axes), _dtype_code(k_cache),
                    _ptr(block_tables), block_tables.shape[1], _ptr(cu_q_lens),
                    _ptr(context_lens), r, hq, hkv, d, bs, float(scale), float(k_scale),
                    float(v_scale))
    return out


def cache_write(k_new, v_new, k_cache, v_cache, slot_mapping,
                k_axes="bhrd", v_axes="bhrd") -> None:
    """Scatter rows of k_new/v_new [T][Hkv][D] into the pools in place ([VE] §3.1)."""
    lib = _load()
    k_new = _c(k_new)
    v_new = _c(v_new)
    slot_mapping = _c(slot_mapping, np.int64)
    assert k_cache.flags.writeable and v_cache.flags.writeable
    t, hkv, d = k_new.shape
    _, _, bs, _ = pool_dims(k_cache, k_axes)
    lib.orc_cache_write(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _strides(k_cache, k_axes),
                        _ptr(v_cache), _strides(v_cache, v_axes), _ptr(slot_mapping), t, hkv, d,
                        bs, k_cache.itemsize)


def swap_blocks(src_k, src_v, dst_k, dst_v, src_dst, k_axes="bhrd", v_axes="bhrd") -> None:
    """Copy whole blocks src_dst[i][0] of the source pools to src_dst[i][1] of
    the destination pools, K and V ([NV] best practice 5, [VI] §2.1 swap)."""
    lib = _load()
    src_dst = _c(src_dst, np.int32).reshape(-1, 2)
    _, hkv, bs, d = pool_dims(src_k, k_axes)
    assert pool_dims(dst_k, k_axes)[1:] == (hkv, bs, d) and src_k.itemsize == dst_k.itemsize
    lib.orc_swap_blocks(_ptr(src_k), _strides(src_k, k_axes), _ptr(src_v),
                        _strides(src_v, v_axes), _ptr(dst_k), _strides(dst_k, k_axes),
                        _ptr(dst_v), _strides(dst_v, v_axes), _ptr(src_dst), src_dst.shape[0],
                        hkv, d, bs, src_k.itemsize)


def copy_blocks(k_cache, v_cache, src_dst, k_axes="bhrd", v_axes="bhrd") -> None:
    """Copy whole blocks src -> dst for K and V in place ([VI] §2.1, COW)."""
    lib = _load()
    src_dst = _c(src_dst, np.int32).reshape(-1, 2)
    _, hkv, bs, d = pool_dims(k_cache, k_axes)
    lib.orc_copy_blocks(_ptr(k_cache), _strides(k_cache, k_axes), _ptr(v_cache),
                        _strides(v_cache, v_axes), _ptr(src_dst), src_dst.shape[0], hkv, d, bs,
                        k_cache.itemsize)

"""C-ABI boundary checks that need no GPU: the library loads, exports every
declared symbol, and rejects bad arguments before enqueuing anything."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_417_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
lib = pa.lib()

FAKE = ctypes.c_void_p(1 << 20)  # aligned, non-NULL; never dereferenced on these paths
MISALIGNED = ctypes.c_void_p((1 << 20) + 4)
NULL = None
STREAM = None


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 19
    for name in syms:
        assert hasattr(lib, name), name
    assert sorted(pa.EXPORTED) == syms


def decode_args(**over):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, tables=FAKE, stride=8, lens=FAKE, S=2, Hq=8, Hkv=8,
             D=128, BS=16, NB=64, scale=0.1, maxlen=100, ps=0, ws=NULL, wsb=0,
             dtype=pa.PA_DTYPE_BF16)
    a.update(over)
    return (a["out"], a["q"], a["k"], a["v"], a["tables"], a["stride"], a["lens"], a["S"], a["Hq"],
            a["Hkv"], a["D"], a["BS"], a["NB"], a["scale"], a["maxlen"], a["ps"], a["ws"],
            a["wsb"], a["dtype"], STREAM)


@pytest.mark.parametrize("over,status", [
    (dict(Hq=6, Hkv=4), pa.PA_ERR_INVALID_ARG),
    (dict(Hq=68, Hkv=4), pa.PA_ERR_UNSUPPORTED),  # group 17
    (dict(D=96), pa.PA_ERR_UNSUPPORTED),
    (dict(BS=8), pa.PA_ERR_UNSUPPORTED),
    (dict(dtype=7), pa.PA_ERR_INVALID_ARG),
    (dict(ps=48), pa.PA_ERR_INVALID_ARG),
    (dict(BS=64, ps=32), pa.PA_ERR_INVALID_ARG),
    (dict(q=NULL), pa.PA_ERR_INVALID_ARG),
    (dict(k=MISALIGNED), pa.PA_ERR_INVALID_ARG),
    (dict(stride=0), pa.PA_ERR_INVALID_ARG),
    (dict(maxlen=-1), pa.PA_ERR_INVALID_ARG),
    (dict(S=-1), pa.PA_ERR_INVALID_ARG),
    (dict(NB=0), pa.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), pa.PA_ERR_INVALID_ARG),
    (dict(maxlen=5000), pa.PA_ERR_INVALID_ARG),  # needs a split-K workspace, none given
])
def test_decode_rejects(over, status):
    assert lib.pa_decode(*decode_args(**over)) == status
    assert lib.pa_last_error()


def test_decode_ex_flags():
    args = list(decode_args(S=0, out=NULL, q=NULL, tables=NULL, lens=NULL))
    assert lib.pa_decode_ex(*args[:-1], pa.PA_DECODE_KV_REUSE, STREAM) == pa.PA_OK
    assert lib.pa_decode_ex(*args[:-1], 0, STREAM) == pa.PA_OK
    assert lib.pa_decode_ex(*args[:-1], 6, STREAM) == pa.PA_ERR_INVALID_ARG
    assert b"flags" in lib.pa_last_error()


def test_decode_workspace_too_small_and_sizes():
    need = pa.pa_decode_workspace_size(2, 8, 8, 128, 16, 5000, 512)
    assert need > 0
    assert lib.pa_decode(*decode_args(maxlen=5000, ps=512, ws=FAKE, wsb=need - 1)) == \
        pa.PA_ERR_INVALID_ARG
    assert pa.pa_decode_workspace_size(2, 8, 8, 128, 16, 512, 512) == 0
    # rows * (2 + D) floats, the (m, l) part rounded up to 256 bytes
    rows = 2 * 8 * 10
    assert need == (rows * 8 + 255) // 256 * 256 + rows * 128 * 4


def test_default_partition_is_a_multiple_of_step_and_block():
    for bs in (16, 32, 64, 128):
        for s, hkv, maxlen in ((64, 32, 4096), (4, 8, 201), (8, 8, 32768), (1, 1, 10)):
            ps = pa.pa_decode_default_partition(s, hkv, bs, maxlen)
            assert ps % 32 == 0 and ps % bs == 0 and 32 <= ps <= 4096
    # Many (sequence, kv head) pairs keep 512; a few long contexts grow the
    # partition while the grid keeps >= 1024 waves; short ones shrink it; a
    # longest context of 16 partitions or more grows it (to 4096 at most)
    # while the grid keeps >= 512 waves.
    assert pa.pa_decode_default_partition(64, 32, 16, 4096) == 512
    assert pa.pa_decode_default_partition(128, 8, 16, 8192) == 1024  # at most 16 partitions
    assert pa.pa_decode_default_partition(8, 8, 128, 32768) == 4096  # 64 pairs x 8 partitions
    assert pa.pa_decode_default_partition(1, 32, 16, 32768) == 2048  # keeps 512 waves
    assert pa.pa_decode_default_partition(4, 8, 16, 201) == 32
    assert pa.pa_decode_default_partition(4, 8, 128, 201) == 128


def test_decode_zero_sequences_is_a_no_op():
    assert lib.pa_decode(*decode_args(S=0, out=NULL, q=NULL, tables=NULL, lens=NULL)) == pa.PA_OK


def test_cache_write_and_copy_reject():
    cw = lib.pa_cache_write
    assert cw(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 96, 16, 64, 1, STREAM) == pa.PA_ERR_UNSUPPORTED
    assert cw(FAKE, FAKE, FAKE, FAKE, NULL, 4, 8, 128, 16, 64, 1, STREAM) == pa.PA_ERR_INVALID_ARG
    assert cw(MISALIGNED, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 64, 1, STREAM) == \
        pa.PA_ERR_INVALID_ARG
    assert cw(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 8, 128, 16, 64, 1, STREAM) == pa.PA_ERR_INVALID_ARG
    assert cw(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 16, 64, 9, STREAM) == pa.PA_ERR_INVALID_ARG
    assert cw(NULL, NULL, FAKE, FAKE, NULL, 0, 8, 128, 16, 64, 1, STREAM) == pa.PA_OK
    cb = lib.pa_copy_blocks
    assert cb(FAKE, FAKE, NULL, 3, 8, 128, 16, 64, 1, STREAM) == pa.PA_ERR_INVALID_ARG
    assert cb(FAKE, FAKE, FAKE, 3, 8, 128, 12, 64, 1, STREAM) == pa.PA_ERR_UNSUPPORTED
    assert cb(FAKE, FAKE, NULL, 0, 8, 128, 16, 64, 1, STREAM) == pa.PA_OK


def test_read_stream_rejects():
    rs = lib.pa_read_stream
    assert rs(NULL, 64, FAKE, STREAM) == pa.PA_ERR_INVALID_ARG
    assert rs(FAKE, 64, NULL, STREAM) == pa.PA_ERR_INVALID_ARG
    assert rs(MISALIGNED, 64, FAKE, STREAM) == pa.PA_ERR_INVALID_ARG
    assert rs(FAKE, 64, ctypes.c_void_p((1 << 20) + 2), STREAM) == \
        pa.PA_ERR_INVALID_ARG
    assert rs(FAKE, 24, FAKE, STREAM) == pa.PA_ERR_INVALID_ARG


def test_prefill_rejects():
    pf = lib.pa_prefill_chunk

    def call(**o):
        a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, t=FAKE, stride=40, cu=FAKE, lens=FAKE, R=4,
                 T=2048, mq=512, mc=4608, Hq=32, Hkv=8, D=128, BS=128, NB=8192, scale=0.08,
                 dtype=pa.PA_DTYPE_BF16)
        a.update(o)
        return pf(a["out"], a["q"], a["k"], a["v"], a["t"], a["stride"], a["cu"], a["lens"],
                  a["R"], a["T"], a["mq"], a["mc"], a["Hq"], a["Hkv"], a["D"], a["BS"], a["NB"],
                  a["scale"], a["dtype"], STREAM)

    assert call(dtype=pa.PA_DTYPE_F32) == pa.PA_ERR_UNSUPPORTED
    assert call(Hq=30) == pa.PA_ERR_INVALID_ARG
    assert call(cu=NULL) == pa.PA_ERR_INVALID_ARG
    assert call(D=80) == pa.PA_ERR_UNSUPPORTED
    assert call(R=-1) == pa.PA_ERR_INVALID_ARG
    assert call(R=0) == pa.PA_OK


def test_error_text_is_thread_local_and_cleared():
    lib.pa_decode(*decode_args(D=96))
    assert b"head_dim" in lib.pa_last_error()
    assert lib.pa_decode(*decode_args(S=0, out=NULL, q=NULL, tables=NULL, lens=NULL)) == pa.PA_OK
    assert lib.pa_last_error() == b""


def grouped_args(offsets=FAKE, seq_group=FAKE, shared=FAKE, ngroups=1, gmax=8, flags=0, **over):
    a = list(decode_args(**over))
    dtype = a[18]
    return tuple(a[:16]) + (offsets, seq_group, shared, ngroups, gmax, a[16], a[17], dtype,
                            flags, STREAM)


@pytest.mark.parametrize("kw,status", [
    (dict(ngroups=-1), pa.PA_ERR_INVALID_ARG),
    (dict(offsets=NULL), pa.PA_ERR_INVALID_ARG),
    (dict(seq_group=NULL), pa.PA_ERR_INVALID_ARG),
    (dict(shared=NULL), pa.PA_ERR_INVALID_ARG),
    (dict(gmax=0), pa.PA_ERR_INVALID_ARG),
    (dict(offsets=MISALIGNED), pa.PA_ERR_INVALID_ARG),
    (dict(flags=4), pa.PA_ERR_INVALID_ARG),
    (dict(dtype=pa.PA_DTYPE_F32), pa.PA_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), pa.PA_ERR_INVALID_ARG),
])
def test_decode_grouped_rejects(kw, status):
    assert lib.pa_decode_grouped(*grouped_args(**kw)) == status
    assert lib.pa_last_error()


def test_decode_grouped_workspace_holds_one_more_partition():
    """A grouped call may split a member at its group's shared region: one
    partition more per (sequence, head) row than pa_decode's; a workspace
    sized for pa_decode is refused (nothing is launched on that path)."""
    plain = pa.pa_decode_workspace_size(2, 8, 8, 128, 16, 5000, 512)
    need = pa.pa_decode_grouped_workspace_size(2, 8, 8, 128, 16, 5000, 512)
    rows = 2 * 8 * 11  # ceil(5000 / 512) + 1 partitions
    assert need == (rows * 8 + 255) // 256 * 256 + rows * 128 * 4 and need > plain
    rows = 2 * 8 * 2  # one partition, and one for a split member
    assert pa.pa_decode_grouped_workspace_size(2, 8, 8, 128, 16, 512, 512) == \
        (rows * 8 + 255) // 256 * 256 + rows * 128 * 4
    assert pa.pa_decode_grouped_workspace_size(0, 8, 8, 128, 16, 512, 512) == 0
    with pytest.raises(pa.PAError):
        pa.pa_decode_grouped_workspace_size(2, 8, 8, 128, 16, -1, 512)
    assert lib.pa_decode_grouped(*grouped_args(maxlen=5000, ps=512, ws=FAKE, wsb=plain)) == \
        pa.PA_ERR_INVALID_ARG
    assert b"workspace" in lib.pa_last_error()


def test_decode_grouped_empty_batch_and_no_groups_are_ok():
    none = dict(S=0, out=NULL, q=NULL, tables=NULL, lens=NULL)
    assert lib.pa_decode_grouped(*grouped_args(**none)) == pa.PA_OK
    assert lib.pa_decode_grouped(*grouped_args(offsets=NULL, seq_group=NULL, shared=NULL,
                                               ngroups=0, gmax=0, **none)) == pa.PA_OK

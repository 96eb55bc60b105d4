"""GPU parity of pa_cache_write and pa_decode against the fp64 oracle.

Bars: cache writes bit-exact; attention max |device - oracle| <= 2e-3 (bf16
KV, fp32 accumulation).  Invariants that must hold bit for bit on the device:
block permutation, shared vs duplicated storage, context length 1 = V,
run-to-run determinism.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from oracle.allocator_model import AllocatorModel
from paged_helpers import chunked_checksum, host_bits, oracle_decode_all, oracle_decode_rows

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def pa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_417_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_decode(pa, case, ps=0, lengths=None, tables=None, q=None, valu=False):
    sh = case.shape
    lens = case.lengths if lengths is None else lengths
    tabs = case.tables if tables is None else tables
    dev = case.k_pool.device
    q = case.q if q is None else q
    maxlen = int(max(lens)) if len(lens) else 0
    t_dev = torch.as_tensor(tabs, dtype=torch.int32, device=dev)
    l_dev = torch.as_tensor(lens, dtype=torch.int32, device=dev)
    out = torch.full((len(lens), sh.num_q_heads, sh.head_dim), 7.0, device=dev)
    ws = pa.decode_workspace(len(lens), sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                             sh.block_size, maxlen, ps, dev)
    pa.pa_decode(out, q, case.k_pool, case.v_pool, t_dev, l_dev, sh.scale, maxlen, ps, ws,
                 valu=valu)
    torch.cuda.synchronize()
    return out


def check_rows(pa, case, out, rows, lengths=None, tables=None):
    sh = case.shape
    lens = case.lengths if lengths is None else lengths
    tabs = case.tables if tables is None else tables
    ref = oracle_decode_rows(case.q, case.k_pool, case.v_pool, tabs, lens, rows, sh.block_size,
                             sh.scale, case.k_axes, case.v_axes)
    got = out[torch.as_tensor(list(rows), device=out.device)].double().cpu().numpy()
    err = np.abs(got - ref).max() if ref.size else 0.0
    assert np.isfinite(got).all()
    assert err <= TOL, f"max abs err {err}"
    return err


def small_case(pa, dtype, hq, hkv, d, bs, lengths, seed=1234, nb=None):
    sh = wl.DecodeShape("custom", len(lengths), hq, hkv, d, bs, 0, dtype, seed)
    need = sum(wl.blocks_needed(L, bs) for L in lengths) + 8
    return wl.make_decode_case(sh, "cuda", pa.K_AXES, pa.V_AXES, lengths=lengths,
                               num_blocks=nb or need)


# ---------------------------------------------------------------------------
# tiny fp32 batch, end to end through the allocator, cache write and decode


def test_tiny_f32_end_to_end(pa):
    sh = wl.TINY_F32
    say("case tiny_f32 end-to-end")
    dev = "cuda"
    rng = np.random.default_rng(sh.seed)
    order = rng.permutation(sh.num_blocks)
    alloc = pa.Allocator(sh.num_blocks, sh.block_size, free_order=order)
    model = AllocatorModel(sh.num_blocks, sh.block_size, free_order=order)
    lens0 = wl.draw_lengths(sh, rng)
    ids = list(range(sh.num_seqs))
    for s in ids:
        alloc.create(s)
        model.create(s)
    gen = wl.make_generator(sh.seed, dev)
    kshape, vshape = pa.kv_cache_shapes(sh.num_blocks, sh.num_kv_heads, sh.block_size,
                                        sh.head_dim)
    k_pool = torch.full(kshape, float("nan"), device=dev)
    v_pool = torch.full(vshape, float("nan"), device=dev)
    k_host = host_bits(k_pool).copy()
    v_host = host_bits(v_pool).copy()

    def step(n_tokens):
        slots, pairs = alloc.batch_append(ids, n_tokens)
        want = []
        for s, n in zip(ids, n_tokens):
            sl, pr = model.append(s, int(n))
            assert pr == []
            want += sl
        assert list(slots) == want  # bit-exact slot assignment
        T = int(sum(n_tokens))
        k_new = wl.randn((T, sh.num_kv_heads, sh.head_dim), torch.float32, gen, dev)
        v_new = wl.randn((T, sh.num_kv_heads, sh.head_dim), torch.float32, gen, dev)
        pa.pa_cache_write(k_new, v_new, k_pool, v_pool,
                          torch.as_tensor(slots, dtype=torch.int64, device=dev))
        oracle.cache_write(host_bits(k_new), host_bits(v_new), k_host, v_host,
                           np.asarray(want, dtype=np.int64), pa.K_AXES, pa.V_AXES)
        torch.cuda.synchronize()
        # whole pools, bit for bit (NaN poison included)
        assert (host_bits(k_pool).view(np.uint32) == k_host.view(np.uint32)).all()
        assert (host_bits(v_pool).view(np.uint32) == v_host.view(np.uint32)).all()
        tables = np.zeros((sh.num_seqs, 16), dtype=np.int32)
        for s in ids:
            tables[s, :len(model.tables[s])] = model.tables[s]
        lens = np.array([model.lengths[s] for s in ids], dtype=np.int32)
        dt, dl = alloc.batch_tables(ids, 16)
        assert (dt[:, :] == tables).all() and (dl == lens).all()
        q = wl.randn((sh.num_seqs, sh.num_q_heads, sh.head_dim), torch.float32, gen, dev)
        for ps in (0, 32, 64, 256):
            out = torch.empty((sh.num_seqs, sh.num_q_heads, sh.head_dim), device=dev)
            maxlen = int(lens.max())
            ws = pa.decode_workspace(sh.num_seqs, sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                                     sh.block_size, maxlen, ps, dev)
            pa.pa_decode(out, q, k_pool, v_pool, torch.as_tensor(tables, device=dev),
                         torch.as_tensor(lens, device=dev), sh.scale, maxlen, ps, ws)
            torch.cuda.synchronize()
            ref = oracle.decode(host_bits(q), k_host, v_host, tables, lens, sh.scale,
                                pa.K_AXES, pa.V_AXES)
            err = np.abs(out.double().cpu().numpy() - ref).max()
            say(f"  lens {list(lens)} ps {ps} max err {err:.3e}")
            assert err <= 1e-5  # fp32 inputs: fp32 rounding only
        return lens

    lens = step(lens0)
    assert [len(model.tables[s]) for s in ids] == [2, 4, 7, 13]
    lens = step(np.ones(sh.num_seqs, dtype=np.int32))
    assert list(lens) == [18, 65, 101, 201]
    assert alloc.stats()["num_used"] == 27


# ---------------------------------------------------------------------------
# shapes, edge lengths, partitions


EDGE = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512,
        513, 700, 1023, 1024, 1025]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_decode_edge_lengths(pa, dtype, d, bs):
    hq, hkv = (8, 2) if bs in (16, 64) else (4, 4)
    say(f"case edge dtype={dtype} d={d} bs={bs} hq={hq} hkv={hkv}")
    case = small_case(pa, dtype, hq, hkv, d, bs, EDGE, seed=17 * d + bs)
    for ps in (0, max(32, bs), 256 if bs <= 128 else bs):
        out = run_decode(pa, case, ps=ps)
        check_rows(pa, case, out, range(len(EDGE)))
        assert (out[0] == 0).all()  # empty context: zero row


@pytest.mark.parametrize("d,bs,hq,hkv", [(128, 16, 32, 32), (128, 128, 32, 8), (64, 32, 8, 1)])
def test_valu_kernel_on_bf16_matches_oracle_and_matrix_core(pa, d, bs, hq, hkv):
    """PA_DECODE_VALU: the vector-ALU kernel on bf16 caches, a second device
    implementation, within the bar of the oracle and within fp32 rounding of
    the matrix-core kernel."""
    say(f"case valu bf16 d={d} bs={bs} hq={hq} hkv={hkv}")
    case = small_case(pa, "bf16", hq, hkv, d, bs, EDGE, seed=3 * d + bs + hq)
    for ps in (0, 256):
        out = run_decode(pa, case, ps=ps, valu=True)
        check_rows(pa, case, out, range(len(EDGE)))
        ref = run_decode(pa, case, ps=ps)
        assert (out - ref).abs().max().item() <= 1e-5
        assert (out[0] == 0).all()


def test_valu_flag_is_refused_where_it_has_no_kernel(pa):
    case = small_case(pa, "bf16", 8, 2, 128, 16, [40, 17], seed=4)
    dev = "cuda"
    t_dev = torch.as_tensor(case.tables, device=dev)
    l_dev = torch.as_tensor(case.lengths, device=dev)
    out = torch.empty((2, 8, 128), device=dev)
    grp = [torch.as_tensor(a, device=dev) for a in (np.array([0, 2], np.int32),
                                                      np.array([0, 0], np.int32),
                                                      np.array([2], np.int32))]
    import ctypes
    lib = pa.lib()
    st = lib.pa_decode_grouped(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(case.q.data_ptr()),
        ctypes.c_void_p(case.k_pool.data_ptr()), ctypes.c_void_p(case.v_pool.data_ptr()),
        ctypes.c_void_p(t_dev.data_ptr()), t_dev.shape[1], ctypes.c_void_p(l_dev.data_ptr()),
        2, 8, 2, 128, 16, case.k_pool.shape[0], 0.1, 40, 0, ctypes.c_void_p(grp[0].data_ptr()),
        ctypes.c_void_p(grp[1].data_ptr()), ctypes.c_void_p(grp[2].data_ptr()), 1, 2, None, 0,
        pa.PA_DTYPE_BF16, pa.PA_DECODE_VALU, None)
    assert st == pa.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_decode_group_sizes(pa, g):
    hkv = 2
    say(f"case group g={g}")
    lens = [1, 40, 333, 1000]
    case = small_case(pa, "bf16", g * hkv, hkv, 128, 16, lens, seed=99 + g)
    out = run_decode(pa, case)
    check_rows(pa, case, out, range(len(lens)))


# ---------------------------------------------------------------------------
# bit-identical invariants


def test_block_permutation_is_bit_identical(pa):
    say("case permutation")
    lens = [37, 500, 1024, 3]
    case = small_case(pa, "bf16", 8, 2, 128, 16, lens, seed=5)
    out1 = run_decode(pa, case)
    # move every block to a new physical id (a random permutation of the pool)
    nb = case.k_pool.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(1)).to(case.k_pool.device)
    k2 = torch.empty_like(case.k_pool)
    v2 = torch.empty_like(case.v_pool)
    k2[perm] = case.k_pool
    v2[perm] = case.v_pool
    t2 = perm.cpu().numpy()[case.tables].astype(np.int32)
    case2 = wl.DecodeCase(case.shape, case.lengths, case.perm, t2, case.q, k2, v2, case.k_axes,
                          case.v_axes)
    out2 = run_decode(pa, case2)
    assert torch.equal(out1, out2)
    out3 = run_decode(pa, case)
    assert torch.equal(out1, out3)  # run to run


def test_kv_reuse_flag_is_bit_identical(pa):
    """The cache policy changes how K/V are loaded, never the result."""
    say("case kv reuse flag")
    for bs in (16, 128):
        case = small_case(pa, "bf16", 8, 2, 128, bs, [37, 500, 1024, 3, 2049], seed=6 + bs)
        sh = case.shape
        dev = "cuda"
        lens = case.lengths
        maxlen = int(max(lens))
        t_dev = torch.as_tensor(case.tables, device=dev)
        l_dev = torch.as_tensor(lens, device=dev)
        ws = pa.decode_workspace(len(lens), 8, 2, 128, bs, maxlen, 0, dev)
        outs = []
        for reuse in (False, True):
            out = torch.empty((len(lens), 8, 128), device=dev)
            pa.pa_decode(out, case.q, case.k_pool, case.v_pool, t_dev, l_dev, sh.scale, maxlen, 0,
                         ws, kv_reuse=reuse)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        check_rows(pa, case, outs[1], range(len(lens)))


def test_context_one_returns_v_exactly(pa):
    say("case len1")
    for dtype in ("bf16", "f32"):
        case = small_case(pa, dtype, 8, 2, 128, 16, [1, 1, 1], seed=8)
        out = run_decode(pa, case)
        for s in range(3):
            b = int(case.tables[s][0])
            v0 = case.v_pool[b, :, :, 0].float()  # [Hkv][D], row 0 of the block
            want = v0.repeat_interleave(4, dim=0)
            assert torch.equal(out[s], want)


def test_shared_blocks_bit_identical_to_duplicated(pa):
    """Sequences whose tables point at one physical copy of a prefix give
    bit-identical results to private copies of it."""
    say("case shared vs duplicated")
    lens = [16 * 20 + 5, 16 * 20 + 9]
    case = small_case(pa, "bf16", 4, 4, 128, 16, lens, seed=21)
    # copy sequence 0's first 20 blocks' content into sequence 1's first 20
    t = case.tables
    src = torch.as_tensor(t[0, :20].astype(np.int64), device="cuda")
    dst = torch.as_tensor(t[1, :20].astype(np.int64), device="cuda")
    case.k_pool[dst] = case.k_pool[src]
    case.v_pool[dst] = case.v_pool[src]
    dup = run_decode(pa, case)
    shared_t = t.copy()
    shared_t[1, :20] = t[0, :20]
    case.k_pool[dst] = float("nan")
    case.v_pool[dst] = float("nan")
    shared = run_decode(pa, case, tables=shared_t)
    assert torch.equal(dup, shared)


def test_partition_size_invariance(pa):
    say("case partition invariance")
    lens = [4000, 2500, 129, 700]
    case = small_case(pa, "bf16", 8, 8, 128, 16, lens, seed=33)
    outs = [run_decode(pa, case, ps=ps) for ps in (32, 64, 512, 4096)]
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 1e-5


def test_bad_table_entry_and_length_give_nan_rows(pa):
    say("case bad inputs")
    lens = [100, 100, 100]
    case = small_case(pa, "bf16", 4, 4, 128, 16, lens, seed=3)
    t = case.tables.copy()
    t[1, 2] = case.k_pool.shape[0] + 5  # out of the pool
    out = run_decode(pa, case, tables=t)
    assert torch.isnan(out[1]).all()
    assert torch.isfinite(out[0]).all() and torch.isfinite(out[2]).all()
    # a length above max_context_len
    dev = "cuda"
    sh = case.shape
    out2 = torch.zeros((3, 4, 128), device=dev)
    l_dev = torch.as_tensor([100, 90, 100], dtype=torch.int32, device=dev)
    pa.pa_decode(out2, case.q, case.k_pool, case.v_pool,
                 torch.as_tensor(case.tables, device=dev), l_dev, sh.scale, 95, 0,
                 pa.decode_workspace(3, 4, 4, 128, 16, 95, 0, dev))
    torch.cuda.synchronize()
    assert torch.isnan(out2[0]).all() and torch.isnan(out2[2]).all()
    assert torch.isfinite(out2[1]).all()


@pytest.mark.parametrize("ps", [0, 256, 512])
def test_bad_block_inside_a_split_sequence_gives_nan_row(pa, ps):
    """A table entry outside the pool in one partition of a sequence split
    over several partitions: that partition's partials are NaN and the
    reduce carries them into the whole row; every other sequence keeps its
    result bit for bit."""
    say(f"case bad block in a split sequence ps={ps}")
    lens = [3000, 100, 2500, 4096]
    case = small_case(pa, "bf16", 8, 2, 128, 16, lens, seed=31)
    clean = run_decode(pa, case, ps=ps)
    t = case.tables.copy()
    t[0, 100] = case.k_pool.shape[0] + 7  # block 100: tokens 1600..1615, an inner partition
    t[3, 255] = -3                         # the last block of the longest sequence
    out = run_decode(pa, case, ps=ps)
    out_bad = run_decode(pa, case, ps=ps, tables=t)
    assert torch.equal(out, clean)
    assert torch.isnan(out_bad[0]).all() and torch.isnan(out_bad[3]).all()
    assert torch.equal(out_bad[1], clean[1]) and torch.equal(out_bad[2], clean[2])
    check_rows(pa, case, clean, range(len(lens)))


# ---------------------------------------------------------------------------
# the named batches at full size: every row against the oracle


@pytest.mark.parametrize("name,ps,valu", [("mha_7b", 0, False), ("gqa", 0, False),
                                          ("gqa", -1, False), ("mixed", 0, False),
                                          ("mixed", 512, False), ("mha_7b", 0, True)])
def test_full_size_batches(pa, name, ps, valu):
    """The 7B-shaped (64 sequences), grouped-query (128) and long-context
    (8 x 32768) batches at full size, in the launch configuration the
    benchmark times (the library's default partitions; the grouped-query
    batch also at the size pa_decode_partition_for_lengths picks from its
    lengths, ps=-1 here; the long-context batch also at 512-token
    partitions): every row of every sequence against the fp64 oracle, run
    on the host threads.  The 7B-shaped batch also on the vector-ALU kernel
    (PA_DECODE_VALU)."""
    sh = wl.SHAPES[name]
    case = wl.make_decode_case(sh, "cuda", pa.K_AXES, pa.V_AXES)
    if ps < 0:
        ps = pa.decode_partition_for_lengths(case.lengths, sh.num_kv_heads, sh.block_size,
                                             int(max(case.lengths)))
    say(f"case full-size {name}: S={sh.num_seqs} Hq={sh.num_q_heads} Hkv={sh.num_kv_heads} "
        f"BS={sh.block_size} NB={sh.num_blocks} ps={ps} valu={valu}")
    out = run_decode(pa, case, ps=ps, valu=valu)
    assert torch.isfinite(out).all()
    ref = oracle_decode_all(case.q, case.k_pool, case.v_pool, case.tables, case.lengths,
                            sh.block_size, sh.scale, case.k_axes, case.v_axes)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    say(f"  all {len(case.lengths)} rows max err {err:.3e}")
    assert err <= TOL, f"max abs err {err}"
    del case
    torch.cuda.empty_cache()


def test_cache_write_full_pool_bit_exact(pa):
    """64 new tokens into the 200,000-block pool: the written rows equal the
    input and no other byte of either pool changes."""
    sh = wl.MHA_7B
    say("case cache write full pool")
    dev = "cuda"
    kshape, vshape = pa.kv_cache_shapes(sh.num_blocks, sh.num_kv_heads, sh.block_size,
                                        sh.head_dim)
    k_pool = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
    before = (chunked_checksum(k_pool), chunked_checksum(v_pool))
    rng = np.random.default_rng(sh.seed)
    blocks = rng.choice(sh.num_blocks, size=64, replace=False)
    offs = rng.integers(0, sh.block_size, size=64)
    slots = blocks.astype(np.int64) * sh.block_size + offs
    slots[5] = -1  # skipped
    gen = wl.make_generator(sh.seed, dev)
    k_new = wl.randn((64, sh.num_kv_heads, sh.head_dim), torch.bfloat16, gen, dev)
    v_new = wl.randn((64, sh.num_kv_heads, sh.head_dim), torch.bfloat16, gen, dev)
    pa.pa_cache_write(k_new, v_new, k_pool, v_pool, torch.as_tensor(slots, device=dev))
    torch.cuda.synchronize()
    # oracle on the touched blocks only
    idx = torch.as_tensor(blocks, device=dev)
    k_sub = host_bits(torch.full_like(k_pool[idx], float("nan")))
    v_sub = host_bits(torch.full_like(v_pool[idx], float("nan")))
    sub_slots = np.arange(64, dtype=np.int64) * sh.block_size + offs
    sub_slots[5] = -1
    oracle.cache_write(host_bits(k_new), host_bits(v_new), k_sub, v_sub, sub_slots, pa.K_AXES,
                       pa.V_AXES)
    assert (host_bits(k_pool[idx]) == k_sub).all()
    assert (host_bits(v_pool[idx]) == v_sub).all()
    # restore the touched blocks to poison: the pools must match the start
    k_pool[idx] = float("nan")
    v_pool[idx] = float("nan")
    assert (chunked_checksum(k_pool), chunked_checksum(v_pool)) == before


@pytest.mark.parametrize("big", [False, True])
@pytest.mark.parametrize("dtype,d,bs", [("bf16", 128, 16), ("bf16", 64, 128), ("f32", 64, 16),
                                         ("f32", 128, 32)])
def test_cache_write_runs_bit_exact(pa, dtype, d, bs, big):
    """Slot patterns of prompt chunks and decode steps mixed in one call:
    aligned runs of consecutive slots, unaligned runs, a run crossing into
    the next block, random slots and skipped (-1) slots.  Small batches and
    batches of hundreds of tokens take different V paths in the library;
    both are checked.  Whole pools are compared with the oracle bit for
    bit."""
    say(f"case cache write runs {dtype} d={d} bs={bs} big={big}")
    dev = "cuda"
    nb, hkv = 48, 4
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kshape, vshape = pa.kv_cache_shapes(nb, hkv, bs, d)
    k_pool = torch.full(kshape, float("nan"), dtype=tdt, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=tdt, device=dev)
    k_host, v_host = host_bits(k_pool).copy(), host_bits(v_pool).copy()
    rng = np.random.default_rng(d + bs)
    blocks = rng.permutation(nb)
    slots = []
    slots += list(range(blocks[0] * bs, blocks[0] * bs + 3 * bs // 2 if bs > 16 else bs))  # aligned run
    slots += list(range(blocks[1] * bs + 3, blocks[1] * bs + bs))  # unaligned start
    slots += list(range(blocks[2] * bs + bs - 5, blocks[2] * bs + bs + 6))  # crosses a block end
    slots += [int(x) for x in rng.choice(np.arange(blocks[5] * bs, blocks[5] * bs + bs), 7,
                                         replace=False)]  # scattered, no run
    slots += [-1, -1, blocks[6] * bs + 1, -1]
    if big:  # whole blocks filled in order, as a prompt chunk does, to past 256 tokens
        j = 7
        while len(slots) < 320:
            slots += list(range(blocks[j] * bs, blocks[j] * bs + bs))
            j += 1
    slots = np.array([sl for sl in slots if sl < nb * bs], dtype=np.int64)
    # keep slots distinct (a slot written twice has no defined winner)
    _, first = np.unique(np.where(slots < 0, -np.arange(len(slots)) - 1, slots), return_index=True)
    slots = slots[np.sort(first)]
    T = len(slots)
    gen = wl.make_generator(d * 7 + bs, dev)
    k_new = wl.randn((T, hkv, d), tdt, gen, dev)
    v_new = wl.randn((T, hkv, d), tdt, gen, dev)
    pa.pa_cache_write(k_new, v_new, k_pool, v_pool, torch.as_tensor(slots, device=dev))
    torch.cuda.synchronize()
    oracle.cache_write(host_bits(k_new), host_bits(v_new), k_host, v_host, slots, pa.K_AXES,
                       pa.V_AXES)
    bits = np.uint16 if dtype == "bf16" else np.uint32
    assert (host_bits(k_pool).view(bits) == k_host.view(bits)).all()
    assert (host_bits(v_pool).view(bits) == v_host.view(bits)).all()


def test_copy_blocks_bit_exact(pa):
    say("case copy blocks")
    case = small_case(pa, "bf16", 8, 8, 128, 16, [300, 200], seed=44)
    nb = case.k_pool.shape[0]
    pairs = np.array([[case.tables[0][3], nb - 2], [case.tables[1][0], nb - 3],
                      [nb + 4, 0]], dtype=np.int32)  # last pair out of range: skipped
    k_host, v_host = host_bits(case.k_pool).copy(), host_bits(case.v_pool).copy()
    pa.pa_copy_blocks(case.k_pool, case.v_pool, torch.as_tensor(pairs, device="cuda"))
    torch.cuda.synchronize()
    oracle.copy_blocks(k_host, v_host, pairs[:2], pa.K_AXES, pa.V_AXES)
    assert (host_bits(case.k_pool) == k_host).all()
    assert (host_bits(case.v_pool) == v_host).all()


@pytest.mark.parametrize("S", [1, 63, 64, 65, 128, 129, 256, 257])
def test_longest_first_grid_edges(pa, S):
    """Batch sizes on both sides of the longest-first grid's 64-sequence chunks
    and of its 256-sequence limit (past which the slot grid runs), lengths
    mixing empty contexts, exactly full partitions, one-token tails and long
    ones, plus two bad lengths: every good row against the oracle, every bad
    row NaN, at the default partition and at 64-token partitions."""
    rng = np.random.default_rng(500 + S)
    maxlen = 700
    lengths = rng.integers(1, maxlen, S)
    for i, v in enumerate([0, 64, 128, 65, 1, maxlen - 1, 512]):
        if i < S:
            lengths[(i * 7) % S] = v
    lengths = [int(x) for x in lengths]
    case = small_case(pa, "bf16", 4, 2, 64, 16, lengths, seed=S)
    sh = case.shape
    dev = "cuda"
    call_lens = list(lengths)
    bad = sorted({S // 3, (2 * S) // 3}) if S >= 3 else []
    if bad:
        call_lens[bad[0]] = -1
        call_lens[bad[-1]] = maxlen + 1
    good = [i for i in range(S) if i not in bad]
    t_dev = torch.as_tensor(case.tables, dtype=torch.int32, device=dev)
    l_dev = torch.as_tensor(call_lens, dtype=torch.int32, device=dev)
    for ps in (0, 64):
        say(f"case longest-first grid S={S} ps={ps}")
        out = torch.full((S, sh.num_q_heads, sh.head_dim), 7.0, device=dev)
        ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                                 sh.block_size, maxlen, ps, dev)
        pa.pa_decode(out, case.q, case.k_pool, case.v_pool, t_dev, l_dev, sh.scale, maxlen, ps,
                     ws)
        torch.cuda.synchronize()
        err = check_rows(pa, case, out, good)
        for b in bad:
            assert torch.isnan(out[b]).all()
        say(f"  {len(good)} rows max err {err:.3e}, {len(bad)} NaN rows")

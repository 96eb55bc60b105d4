"""GPU parity of pa_prefill_chunk against the fp64 oracle, and the mixed
continuous-batching step (cache write of decode tokens and prompt chunks,
then decode and chunked prefill in one iteration).

Bar: max |device - oracle| <= 2e-3 (bf16 K/V/q, fp32 accumulation and
output).  Rows of a chunk are causal: the row at absolute position p sees
keys 0..p of its request.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from paged_helpers import gather_blocks, host_bits, oracle_decode_rows

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


def run_prefill(pa, case, cu=None, ctx=None, max_q_len=None, max_ctx=None):
    sh = case.shape
    dev = case.k_pool.device
    cu = case.cu_q_lens if cu is None else cu
    ctx = case.context_lens if ctx is None else ctx
    qlens = np.diff(cu)
    mq = int(qlens.max()) if max_q_len is None else max_q_len
    mc = int(np.max(ctx)) if max_ctx is None else max_ctx
    out = torch.full((case.q.shape[0], sh.num_q_heads, sh.head_dim), 7.0, device=dev)
    pa.pa_prefill_chunk(out, case.q, case.k_pool, case.v_pool,
                        torch.as_tensor(case.tables, dtype=torch.int32, device=dev),
                        torch.as_tensor(cu, dtype=torch.int32, device=dev),
                        torch.as_tensor(ctx, dtype=torch.int32, device=dev), sh.scale, mq, mc)
    torch.cuda.synchronize()
    return out


def oracle_prefill_all(case):
    rows = list(range(len(case.context_lens)))
    k_sub, v_sub, t_sub, l_sub = gather_blocks(case.k_pool, case.v_pool, case.tables,
                                               case.context_lens, rows, case.shape.block_size)
    return oracle.prefill(host_bits(case.q), k_sub, v_sub, t_sub, case.cu_q_lens, l_sub,
                          case.shape.scale, case.k_axes, case.v_axes)


def oracle_prefill_rows(case, picks):
    """Oracle output for selected (request, row) pairs: each is the 1-row
    chunk at its absolute position p over keys 0..p."""
    sh = case.shape
    out = {}
    for r, i in picks:
        p = int(case.context_lens[r] - case.q_lens[r] + i)
        k_sub, v_sub, t_sub, _ = gather_blocks(case.k_pool, case.v_pool, case.tables[[r]],
                                               [p + 1], [0], sh.block_size)
        qrow = host_bits(case.q[int(case.cu_q_lens[r]) + i:int(case.cu_q_lens[r]) + i + 1])
        out[(r, i)] = oracle.prefill(qrow, k_sub, v_sub, t_sub, np.array([0, 1], np.int32),
                                     np.array([p + 1], np.int32), sh.scale, case.k_axes,
                                     case.v_axes)[0]
    return out


def check_all(case, out):
    ref = oracle_prefill_all(case)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= TOL, f"max abs err {err}"
    return err


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bs", [16, 32, 64, 128])
def test_prefill_shapes(pa, d, bs):
    # (context, new rows): pure prompt, chunk over cache, single row, ragged tails
    ctx = [1, 33, 70, 200, 129, 300]
    ql = [1, 33, 5, 1, 129, 77]
    sh = wl.PrefillShape(num_reqs=len(ctx), num_q_heads=8, num_kv_heads=2, head_dim=d,
                         block_size=bs, seed=1000 + d + bs)
    say(f"case prefill d={d} bs={bs}")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES, context_lens=ctx, q_lens=ql)
    out = run_prefill(pa, case)
    say(f"  max err {check_all(case, out):.3e}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (6, 2), (8, 1), (32, 2), (16, 16)])
def test_prefill_group_sizes(pa, hq, hkv):
    ctx = [150, 64, 400]
    ql = [150, 31, 97]
    sh = wl.PrefillShape(num_reqs=3, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                         block_size=16, seed=77 + hq * 3 + hkv)
    say(f"case prefill group hq={hq} hkv={hkv}")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES, context_lens=ctx, q_lens=ql)
    out = run_prefill(pa, case)
    say(f"  max err {check_all(case, out):.3e}")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.7])
def test_prefill_any_scale(pa, scale):
    """The scale may be negative or zero (scale 0 gives the mean of the
    visible V rows)."""
    ctx, ql = [90, 40, 257], [90, 7, 33]
    sh = wl.PrefillShape(num_reqs=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, seed=61)
    say(f"case prefill scale {scale}")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES, context_lens=ctx, q_lens=ql)
    dev = "cuda"
    out = torch.full((case.q.shape[0], 8, 128), 7.0, device=dev)
    pa.pa_prefill_chunk(out, case.q, case.k_pool, case.v_pool,
                        torch.as_tensor(case.tables, device=dev),
                        torch.as_tensor(case.cu_q_lens, device=dev),
                        torch.as_tensor(case.context_lens, device=dev), scale, max(ql), max(ctx))
    torch.cuda.synchronize()
    rows = list(range(3))
    k_sub, v_sub, t_sub, l_sub = gather_blocks(case.k_pool, case.v_pool, case.tables,
                                               case.context_lens, rows, sh.block_size)
    ref = oracle.prefill(host_bits(case.q), k_sub, v_sub, t_sub, case.cu_q_lens, l_sub, scale,
                         case.k_axes, case.v_axes)
    err = float(np.abs(out.double().cpu().numpy() - ref).max())
    say(f"  max err {err:.3e}")
    assert err <= TOL


def test_prefill_last_row_matches_decode(pa):
    """The last row of a chunk is a decode step over the whole context."""
    sh = wl.PrefillShape(num_reqs=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, seed=5)
    ctx, ql = [300, 45, 1000], [60, 45, 1]
    say("case prefill last row vs decode")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES, context_lens=ctx, q_lens=ql)
    out = run_prefill(pa, case)
    last = torch.as_tensor(case.cu_q_lens[1:] - 1, device="cuda", dtype=torch.long)
    qd = case.q[last].contiguous()
    dec = torch.empty_like(out[last])
    mx = int(max(ctx))
    ws = pa.decode_workspace(3, 8, 2, 128, 16, mx, 0, "cuda")
    pa.pa_decode(dec, qd, case.k_pool, case.v_pool,
                 torch.as_tensor(case.tables, device="cuda"),
                 torch.as_tensor(ctx, dtype=torch.int32, device="cuda"), sh.scale, mx, 0, ws)
    torch.cuda.synchronize()
    # prefill rounds its weights to fp16 (relative 2^-11), decode splits them
    # into bf16 high and low parts: the two meet the oracle's bar, not each
    # other's rounding
    diff = (out[last] - dec).abs().max().item()
    say(f"  max |prefill last row - decode| {diff:.3e}")
    assert diff <= TOL


@pytest.mark.parametrize("mode", ["whole_pool", "one_element", "last_key", "infinite"])
def test_prefill_v_beyond_fp16_range(pa, mode):
    """V elements that fp16 cannot hold (beyond 65504, or infinite) send the
    workgroups that stage them through the bf16 high/low walk: the result
    keeps its accuracy relative to the size of V instead of overflowing."""
    ctx, ql = [200, 70, 33], [40, 70, 33]
    sh = wl.PrefillShape(num_reqs=3, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=16, seed=404)
    say(f"case prefill V beyond fp16 range ({mode})")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES, context_lens=ctx, q_lens=ql)
    big = 2.0 ** 20
    if mode == "whole_pool":
        case.v_pool.mul_(big)  # exact in bf16; every used V element is scaled
    elif mode == "last_key":
        # one element of request 0's last key (199): only its last row sees it,
        # the other rows of that row's workgroup meet it with a zero weight
        at = {"b": int(case.tables[0][199 // 16]), "h": 1, "r": 199 % 16, "d": 5}
        case.v_pool[tuple(at[ax] for ax in case.v_axes)] = 3.0e5
    else:
        # one element of request 0's key 3 (seen by every row of request 0)
        at = {"b": int(case.tables[0][0]), "h": 1, "r": 3, "d": 5}  # kv head 1, dim 5
        case.v_pool[tuple(at[ax] for ax in case.v_axes)] = (
            float("inf") if mode == "infinite" else 3.0e5)
    out = run_prefill(pa, case)
    ref = oracle_prefill_all(case)
    got = out.double().cpu().numpy()
    if mode == "infinite":
        # every row of request 0 weighs the infinite element: dim 5 of the
        # query heads of kv head 1 is +inf exactly (the device may give NaN
        # there, where a zero weight part meets the infinity); nothing else
        # is touched
        hmask = np.zeros(got.shape, bool)
        hmask[:40, 4:8, 5] = True
        assert np.isposinf(ref[hmask]).all() and not np.isfinite(got[hmask]).any()
        fin = ~hmask
        err = float(np.abs(got[fin] - ref[fin]).max())
        say(f"  max err outside the infinite column {err:.3e}")
        assert err <= TOL
        return
    assert np.isfinite(got).all()
    if mode == "whole_pool":
        # the same problem with V scaled by 2^20: the error scales with V
        err = float(np.abs(got - ref).max()) / big
        say(f"  max err / 2^20 {err:.3e}")
        assert err <= TOL
        return
    rel = float((np.abs(got - ref) / np.maximum(1.0, np.abs(ref))).max())
    say(f"  max err relative to max(1, |ref|) {rel:.3e}")
    assert rel <= TOL


def test_prefill_determinism_and_permutation(pa):
    sh = wl.PrefillShape(num_reqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         block_size=32, seed=9)
    say("case prefill determinism / permutation")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES, context_lens=[500, 260],
                                q_lens=[200, 260])
    a = run_prefill(pa, case)
    b = run_prefill(pa, case)
    assert torch.equal(a, b)
    nb = case.k_pool.shape[0]
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(2)).to("cuda")
    k2, v2 = torch.empty_like(case.k_pool), torch.empty_like(case.v_pool)
    k2[perm] = case.k_pool
    v2[perm] = case.v_pool
    t2 = perm.cpu().numpy()[case.tables].astype(np.int32)
    case2 = wl.PrefillCase(case.shape, case.context_lens, case.q_lens, case.cu_q_lens,
                           case.perm, t2, case.q, k2, v2, case.k_axes, case.v_axes)
    c = run_prefill(pa, case2)
    assert torch.equal(a, c)


def test_prefill_bad_inputs(pa):
    sh = wl.PrefillShape(num_reqs=3, num_q_heads=4, num_kv_heads=4, head_dim=128,
                         block_size=16, seed=10)
    say("case prefill bad inputs")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES, context_lens=[40, 40, 40],
                                q_lens=[10, 10, 10])
    # request 1: a table entry outside the pool
    t = case.tables.copy()
    t[1, 1] = case.k_pool.shape[0] + 3
    case_t = wl.PrefillCase(case.shape, case.context_lens, case.q_lens, case.cu_q_lens, case.perm,
                            t, case.q, case.k_pool, case.v_pool, case.k_axes, case.v_axes)
    out = run_prefill(pa, case_t)
    assert torch.isnan(out[10:20]).all()
    assert torch.isfinite(out[:10]).all() and torch.isfinite(out[20:]).all()
    # request 2: context shorter than its chunk
    out2 = run_prefill(pa, case, ctx=np.array([40, 40, 5], np.int32))
    assert torch.isnan(out2[20:30]).all() and torch.isfinite(out2[:20]).all()


def test_prefill_full_size_mixed_chunks(pa):
    """Four 512-row chunks over 4096 cached tokens (block 128, 32 q / 8 kv
    heads, head_dim 128): sampled rows against the oracle."""
    sh = wl.MIXED_PREFILL
    say("case prefill full size 4 x 512 over 4096")
    case = wl.make_prefill_case(sh, "cuda", pa.K_AXES, pa.V_AXES)
    out = run_prefill(pa, case)
    assert torch.isfinite(out).all()
    picks = [(0, 0), (0, 511), (1, 1), (1, 255), (2, 128), (2, 383), (3, 31), (3, 510)]
    ref = oracle_prefill_rows(case, picks)
    err = 0.0
    for (r, i), want in ref.items():
        got = out[int(case.cu_q_lens[r]) + i].double().cpu().numpy()
        err = max(err, float(np.abs(got - want).max()))
    say(f"  sampled rows max err {err:.3e}")
    assert err <= TOL


def test_mixed_step_end_to_end(pa):
    """One continuous-batching iteration: 8 decode sequences at 32768 tokens
    (block 128, partitions of 512) and 4 prompt chunks of 512 new tokens over
    4096 cached; the allocator assigns every slot, one pa_cache_write stores
    all 8 + 2048 new K/V rows, then pa_decode and pa_prefill_chunk run on one
    stream.  Sampled rows of both are checked against the oracle; the step
    with the prefill on a second stream gives the same bits."""
    dev = "cuda"
    dsh, psh = wl.MIXED_DECODE, wl.MIXED_PREFILL
    hkv, d, bs = dsh.num_kv_heads, dsh.head_dim, dsh.block_size
    say("case mixed step")
    rng = np.random.default_rng(dsh.seed)
    nb = dsh.num_blocks
    alloc = pa.Allocator(nb, bs, free_order=rng.permutation(nb))
    dec_ids = list(range(8))
    pre_ids = list(range(100, 104))
    for s in dec_ids + pre_ids:
        alloc.create(s)
    kshape, vshape = pa.kv_cache_shapes(nb, hkv, bs, d)
    k_pool = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
    gen = wl.make_generator(dsh.seed, dev)
    # history: 32767 tokens per decode sequence, 4096 cached per prompt
    slots, pairs = alloc.batch_append(dec_ids + pre_ids, [32767] * 8 + [4096] * 4)
    assert len(pairs) == 0
    t = len(slots)
    for lo in range(0, t, 65536):
        hi = min(t, lo + 65536)
        kn = wl.randn((hi - lo, hkv, d), torch.bfloat16, gen, dev)
        vn = wl.randn((hi - lo, hkv, d), torch.bfloat16, gen, dev)
        pa.pa_cache_write(kn, vn, k_pool, v_pool, torch.as_tensor(slots[lo:hi], device=dev))
    # the step: one new token per decode sequence, 512 per prompt chunk
    slots, pairs = alloc.batch_append(dec_ids + pre_ids, [1] * 8 + [512] * 4)
    assert len(slots) == 8 + 2048 and len(pairs) == 0
    kn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    vn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    pa.pa_cache_write(kn, vn, k_pool, v_pool, torch.as_tensor(slots, device=dev))
    dt, dl = alloc.batch_tables(dec_ids, 257)
    pt, pl = alloc.batch_tables(pre_ids, 40)
    assert list(dl) == [32768] * 8 and list(pl) == [4608] * 4
    qd = wl.randn((8, dsh.num_q_heads, d), torch.bfloat16, gen, dev)
    qp = wl.randn((2048, psh.num_q_heads, d), torch.bfloat16, gen, dev)
    out_d = torch.empty((8, dsh.num_q_heads, d), device=dev)
    out_p = torch.empty((2048, psh.num_q_heads, d), device=dev)
    ws = pa.decode_workspace(8, dsh.num_q_heads, hkv, d, bs, 32768, 512, dev)
    cu = np.arange(0, 2049, 512, dtype=np.int32)
    pa.pa_decode(out_d, qd, k_pool, v_pool, torch.as_tensor(dt, device=dev),
                 torch.as_tensor(dl, device=dev), dsh.scale, 32768, 512, ws)
    pa.pa_prefill_chunk(out_p, qp, k_pool, v_pool, torch.as_tensor(pt, device=dev),
                        torch.as_tensor(cu, device=dev), torch.as_tensor(pl, device=dev),
                        psh.scale, 512, 4608)
    torch.cuda.synchronize()
    assert torch.isfinite(out_d).all() and torch.isfinite(out_p).all()
    err_d = 0.0
    for s in (0, 5):
        ref = oracle_decode_rows(qd, k_pool, v_pool, dt, dl, [s], bs, dsh.scale, pa.K_AXES,
                                 pa.V_AXES)
        err_d = max(err_d, float(np.abs(out_d[s].double().cpu().numpy() - ref[0]).max()))
    case = wl.PrefillCase(psh, pl, np.full(4, 512, np.int32), cu, None, pt, qp, k_pool, v_pool,
                          pa.K_AXES, pa.V_AXES)
    ref = oracle_prefill_rows(case, [(0, 0), (1, 300), (3, 511)])
    err_p = max(float(np.abs(out_p[int(cu[r]) + i].double().cpu().numpy() - want).max())
                for (r, i), want in ref.items())
    say(f"  decode err {err_d:.3e} prefill err {err_p:.3e}")
    assert err_d <= TOL and err_p <= TOL

    # the same step with the decode and the prefill on two created streams
    # (both default priority), the prefill's stream waiting for the decode's
    # at its start: bit-identical, repeated
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    dt_d, dl_d = torch.as_tensor(dt, device=dev), torch.as_tensor(dl, device=dev)
    pt_d, pl_d = torch.as_tensor(pt, device=dev), torch.as_tensor(pl, device=dev)
    cu_d = torch.as_tensor(cu, device=dev)
    for rep in range(3):
        out_d2, out_p2 = torch.full_like(out_d, 7.0), torch.full_like(out_p, 7.0)
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(s1)
        pa.pa_decode(out_d2, qd, k_pool, v_pool, dt_d, dl_d, dsh.scale, 32768, 512, ws, stream=s1)
        pa.pa_prefill_chunk(out_p2, qp, k_pool, v_pool, pt_d, cu_d, pl_d, psh.scale, 512, 4608,
                            stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(out_d2, out_d) and torch.equal(out_p2, out_p), rep

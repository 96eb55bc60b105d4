"""Prefix-shared parallel sampling on the GPU: 16 prompts, each forked into 8
samples that share the prompt's blocks through refcounted block tables, then
given private tails of 1..512 tokens.  The prompt's last block is partly
filled and shared, so every sample but the last holder copies it first
(copy-on-write through pa_copy_blocks) before its cache write.

Checks: the copies and writes are bit-exact and leave the shared source
intact; decode over shared tables is bit-identical to decode over private
duplicates of the same content; every row matches the fp64 oracle within
2e-3; forking exactly at a block boundary needs no copy.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from paged_helpers import host_bits, oracle_decode_all

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


def build_shared_batch(pa, sh, plan, dev, pool_blocks):
    """Run the allocator through prompts, forks and tails; write every token's
    K/V.  Returns (alloc, ids, k_pool, v_pool, free_order, cow_pairs)."""
    rng = np.random.default_rng(sh.seed)
    order = rng.permutation(pool_blocks)
    alloc = pa.Allocator(pool_blocks, sh.block_size, free_order=order)
    hkv, d = sh.num_kv_heads, sh.head_dim
    kshape, vshape = pa.kv_cache_shapes(pool_blocks, hkv, sh.block_size, d)
    k_pool = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
    gen = wl.make_generator(sh.seed, dev)
    n_prompts, samples = plan.tail_lens.shape
    prompt_ids = [1000 * i for i in range(n_prompts)]
    for pid in prompt_ids:
        alloc.create(pid)
    slots, pairs = alloc.batch_append(prompt_ids, plan.shared_lens)
    assert len(pairs) == 0
    kn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    vn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    pa.pa_cache_write(kn, vn, k_pool, v_pool, torch.as_tensor(slots, device=dev))
    ids = []
    for pid in prompt_ids:
        ids.append(pid)
        for k in range(1, samples):
            alloc.fork(pid, pid + k)
            ids.append(pid + k)
    tails = plan.tail_lens.reshape(-1)
    slots, pairs = alloc.batch_append(ids, tails)
    if len(pairs):
        pa.pa_copy_blocks(k_pool, v_pool, torch.as_tensor(pairs, device=dev))
    kn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    vn = wl.randn((len(slots), hkv, d), torch.bfloat16, gen, dev)
    pa.pa_cache_write(kn, vn, k_pool, v_pool, torch.as_tensor(slots, device=dev))
    torch.cuda.synchronize()
    return alloc, ids, k_pool, v_pool, order, pairs


def test_prefix_shared_sampling(pa):
    sh = wl.PREFIX_SHARED
    dev = "cuda"
    plan = wl.prefix_plan()
    say(f"case prefix-shared: {plan.tail_lens.shape} samples, shared {list(plan.shared_lens[:4])}..")
    alloc, ids, k_pool, v_pool, order, pairs = build_shared_batch(pa, sh, plan, dev,
                                                                  sh.num_blocks)
    n_prompts, samples = plan.tail_lens.shape
    # one copy per sample except the last holder of each prompt's partial block
    assert len(pairs) == n_prompts * (samples - 1)
    st = alloc.stats()
    assert st["cow_copies"] == n_prompts * (samples - 1)
    full_shared = sum(int(L) // sh.block_size for L in plan.shared_lens)
    assert st["num_shared"] == full_shared
    stride = max(wl.blocks_needed(alloc.length(s), sh.block_size) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    # every sample reads the same physical blocks for its full shared blocks
    for i in range(n_prompts):
        nfull = int(plan.shared_lens[i]) // sh.block_size
        grp = tables[i * samples:(i + 1) * samples, :nfull]
        assert (grp == grp[0]).all()
    # copy sources hold the prompt's partial block unchanged: each copy's
    # first rows equal its source's rows bit for bit
    src = torch.as_tensor(pairs[:, 0].astype(np.int64), device=dev)
    dst = torch.as_tensor(pairs[:, 1].astype(np.int64), device=dev)
    for p, (s_b, d_b) in enumerate(pairs):
        j = int(plan.shared_lens[p // (samples - 1)]) % sh.block_size
        assert torch.equal(k_pool[d_b, :, :j].view(torch.int16), k_pool[s_b, :, :j].view(torch.int16))
        assert torch.equal(v_pool[d_b, :, :, :j].view(torch.int16),
                           v_pool[s_b, :, :, :j].view(torch.int16))
    del src, dst

    gen = wl.make_generator(sh.seed + 7, dev)
    S = len(ids)
    q = wl.randn((S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    maxlen = int(lens.max())
    t_dev = torch.as_tensor(tables, device=dev)
    l_dev = torch.as_tensor(lens, device=dev)
    ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                             maxlen, 0, dev)
    out_shared = torch.empty((S, sh.num_q_heads, sh.head_dim), device=dev)
    pa.pa_decode(out_shared, q, k_pool, v_pool, t_dev, l_dev, sh.scale, maxlen, 0, ws)

    # private duplicates: every table entry of every sequence gets its own
    # fresh block holding a bit copy of the original
    used = st["num_used"]
    fresh = iter(order[used:].tolist())
    dup_tables = np.full_like(tables, sh.num_blocks - 1)
    copy_pairs = []
    for s in range(S):
        for j in range(wl.blocks_needed(int(lens[s]), sh.block_size)):
            b = next(fresh)
            dup_tables[s, j] = b
            copy_pairs.append((int(tables[s, j]), b))
    pa.pa_copy_blocks(k_pool, v_pool, torch.as_tensor(np.asarray(copy_pairs, np.int32), device=dev))
    out_dup = torch.empty_like(out_shared)
    pa.pa_decode(out_dup, q, k_pool, v_pool, torch.as_tensor(dup_tables, device=dev), l_dev,
                 sh.scale, maxlen, 0, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out_shared).all()
    assert torch.equal(out_shared, out_dup)
    say(f"  shared == duplicated bit for bit over {S} sequences, {len(copy_pairs)} blocks")

    # every sequence against the fp64 oracle (the shared blocks are copied
    # to the host once)
    ref = oracle_decode_all(q, k_pool, v_pool, tables, lens, sh.block_size, sh.scale,
                            pa.K_AXES, pa.V_AXES)
    err = float(np.abs(out_shared.double().cpu().numpy() - ref).max())
    say(f"  all {S} rows max err {err:.3e}")
    assert err <= TOL


def test_fork_at_block_boundary_needs_no_copy(pa):
    """Forking right after a 2048-token prompt (128 full blocks) leaves no
    partial shared block: the samples' first appends take fresh blocks."""
    sh = wl.PREFIX_SHARED
    plan = wl.prefix_plan(num_prompts=2, samples=8, fork_offsets=False)
    alloc = pa.Allocator(4096, sh.block_size)
    for i in range(2):
        alloc.create(i * 100)
    alloc.batch_append([0, 100], plan.shared_lens)
    ids = []
    for pid in (0, 100):
        ids.append(pid)
        for k in range(1, 8):
            alloc.fork(pid, pid + k)
            ids.append(pid + k)
    slots, pairs = alloc.batch_append(ids, plan.tail_lens.reshape(-1))
    assert len(pairs) == 0
    assert alloc.stats()["cow_copies"] == 0
    assert alloc.stats()["num_shared"] == 2 * 128


def test_cow_then_write_leaves_other_sharers_intact(pa):
    """Small case with the whole pools on the host: after a fork, copy and
    tail writes, every sequence un-pages (oracle) to its prompt followed by
    its own tail, bit for bit."""
    sh = wl.DecodeShape("cow_small", 4, 4, 2, 64, 16, 64, "bf16", 31)
    dev = "cuda"
    alloc = pa.Allocator(sh.num_blocks, sh.block_size,
                         free_order=np.random.default_rng(3).permutation(sh.num_blocks))
    kshape, vshape = pa.kv_cache_shapes(sh.num_blocks, 2, 16, 64)
    k_pool = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
    gen = wl.make_generator(5, dev)
    alloc.create(0)
    prompt_len = 37
    slots, _ = alloc.append(0, prompt_len)
    kp = wl.randn((prompt_len, 2, 64), torch.bfloat16, gen, dev)
    vp = wl.randn((prompt_len, 2, 64), torch.bfloat16, gen, dev)
    pa.pa_cache_write(kp, vp, k_pool, v_pool, torch.as_tensor(slots, device=dev))
    for c in (1, 2, 3):
        alloc.fork(0, c)
    tails = {0: 5, 1: 20, 2: 1, 3: 11}
    tail_k, tail_v = {}, {}
    for s in (1, 2, 0, 3):  # the parent is not last: it copies too
        slots, pairs = alloc.append(s, tails[s])
        if len(pairs):
            pa.pa_copy_blocks(k_pool, v_pool, torch.as_tensor(pairs, device=dev))
        tail_k[s] = wl.randn((tails[s], 2, 64), torch.bfloat16, gen, dev)
        tail_v[s] = wl.randn((tails[s], 2, 64), torch.bfloat16, gen, dev)
        pa.pa_cache_write(tail_k[s], tail_v[s], k_pool, v_pool, torch.as_tensor(slots, device=dev))
    torch.cuda.synchronize()
    assert alloc.stats()["cow_copies"] == 3
    kh, vh = host_bits(k_pool), host_bits(v_pool)
    for s in range(4):
        table = alloc.block_table(s)
        L = prompt_len + tails[s]
        assert alloc.length(s) == L
        for h in range(2):
            k = oracle.unpage(kh, pa.K_AXES, table, L, h)
            v = oracle.unpage(vh, pa.V_AXES, table, L, h)
            want_k = np.concatenate([oracle.widen(host_bits(kp[:, h])),
                                     oracle.widen(host_bits(tail_k[s][:, h]))])
            want_v = np.concatenate([oracle.widen(host_bits(vp[:, h])),
                                     oracle.widen(host_bits(tail_v[s][:, h]))])
            assert (k == want_k).all() and (v == want_v).all()


def test_prefix_cache_hits_decode_like_fresh_prompts(pa):
    """Requests open with one of four shared system prompts.  A first wave
    (one request per system prompt) is written and released, so its full
    blocks wait in the cache queue; a second wave finds them there
    (pa_seq_create_prefix), writes only its uncached positions, and decodes.
    K/V rows are a function of (system prompt, position) inside the system
    prompt, so reuse is exact.  Decode over the cached tables must equal, bit
    for bit, decode over the same prompts written in full into private blocks
    by an allocator without the cache; every row matches the fp64 oracle."""
    sh = wl.DecodeShape("prefix_cache", 12, 8, 4, 64, 16, 1024, "bf16", 77)
    dev = "cuda"
    plan = wl.chat_plan(num_system=4, requests=12, system_len=300, max_user=200)
    hkv, d, bs = sh.num_kv_heads, sh.head_dim, sh.block_size
    gen = wl.make_generator(sh.seed, dev)
    sys_k = [wl.randn((len(t), hkv, d), torch.bfloat16, gen, dev) for t in plan.system_tokens]
    sys_v = [wl.randn((len(t), hkv, d), torch.bfloat16, gen, dev) for t in plan.system_tokens]
    usr_k = [wl.randn((len(t), hkv, d), torch.bfloat16, gen, dev) for t in plan.user_tokens]
    usr_v = [wl.randn((len(t), hkv, d), torch.bfloat16, gen, dev) for t in plan.user_tokens]

    def rows(r, lo):
        """K/V rows of request r's positions lo.. (system rows, then user rows)."""
        s, n_sys = int(plan.system_of[r]), len(plan.system_tokens[int(plan.system_of[r])])
        ks = torch.cat([sys_k[s], usr_k[r]])[lo:]
        vs = torch.cat([sys_v[s], usr_v[r]])[lo:]
        assert ks.shape[0] == n_sys + len(plan.user_tokens[r]) - lo
        return ks.contiguous(), vs.contiguous()

    def pools():
        kshape, vshape = pa.kv_cache_shapes(sh.num_blocks, hkv, bs, d)
        return (torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev),
                torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev))

    order = np.random.default_rng(sh.seed).permutation(sh.num_blocks)
    cached = pa.Allocator(sh.num_blocks, bs, free_order=order)
    kc, vc = pools()
    cached_tokens = {}
    for wave in (range(4), range(4, 12)):
        for r in wave:
            toks = plan.prompt(r)
            n = cached.create_prefix(r, toks, len(toks) - 1)
            cached_tokens[r] = n
            slots, pairs = cached.append_tokens(r, toks[n:])
            assert len(pairs) == 0
            k, v = rows(r, n)
            pa.pa_cache_write(k, v, kc, vc, torch.as_tensor(slots, device=dev))
        if wave.start == 0:
            for r in wave:
                cached.free(r)
            # every full block of the first wave's prompts stays cached
            assert cached.prefix_stats()["cached_free_blocks"] == sum(
                len(plan.prompt(r)) // bs for r in wave)
    ids = list(range(4, 12))
    st = cached.prefix_stats()
    say(f"case prefix cache: hits {st['hit_blocks']} of {st['queried_blocks']} blocks, "
        f"cached tokens {[cached_tokens[r] for r in ids]}")
    for r in ids:  # every second-wave request reused its system prompt's full blocks
        assert cached_tokens[r] == len(plan.system_tokens[int(plan.system_of[r])]) // bs * bs

    fresh = pa.Allocator(sh.num_blocks, bs, free_order=order)
    kf, vf = pools()
    for r in ids:
        fresh.create(r)
        slots, _ = fresh.append(r, len(plan.prompt(r)))
        k, v = rows(r, 0)
        pa.pa_cache_write(k, v, kf, vf, torch.as_tensor(slots, device=dev))

    stride = max(wl.blocks_needed(len(plan.prompt(r)), bs) for r in ids) + 1
    tc, lc = cached.batch_tables(ids, stride, sh.num_blocks - 1)
    tf, lf = fresh.batch_tables(ids, stride, sh.num_blocks - 1)
    assert (lc == lf).all()
    S = len(ids)
    q = wl.randn((S, sh.num_q_heads, d), torch.bfloat16, wl.make_generator(sh.seed + 1, dev), dev)
    maxlen = int(lc.max())
    ws = pa.decode_workspace(S, sh.num_q_heads, hkv, d, bs, maxlen, 64, dev)
    l_dev = torch.as_tensor(lc, device=dev)
    out_c = torch.empty((S, sh.num_q_heads, d), device=dev)
    out_f = torch.empty_like(out_c)
    pa.pa_decode(out_c, q, kc, vc, torch.as_tensor(tc, device=dev), l_dev, sh.scale, maxlen, 64, ws)
    pa.pa_decode(out_f, q, kf, vf, torch.as_tensor(tf, device=dev), l_dev, sh.scale, maxlen, 64, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(out_c).all()
    assert torch.equal(out_c, out_f)
    ref = oracle_decode_all(q, kc, vc, tc, lc, bs, sh.scale, pa.K_AXES, pa.V_AXES)
    err = float(np.abs(out_c.double().cpu().numpy() - ref).max())
    say(f"  cached == fresh bit for bit over {S} requests; oracle, all rows, err {err:.3e}")
    assert err <= TOL


def _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, groups, ps, max_group):
    """Per-sequence decode (kv reuse) and grouped decode of one batch."""
    dev = "cuda"
    S = q.shape[0]
    maxlen = int(lens.max())
    t_dev = torch.as_tensor(tables, device=dev)
    l_dev = torch.as_tensor(lens, device=dev)
    ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                             maxlen, ps, dev, grouped=True)
    ref = torch.full((S, sh.num_q_heads, sh.head_dim), 7.0, device=dev)
    pa.pa_decode(ref, q, k_pool, v_pool, t_dev, l_dev, sh.scale, maxlen, ps, ws, kv_reuse=True)
    off, sg, shd = (torch.as_tensor(a, device=dev) for a in groups)
    got = torch.full_like(ref, 7.0)
    pa.pa_decode_grouped(got, q, k_pool, v_pool, t_dev, l_dev, sh.scale, maxlen, off, sg, shd,
                         max_group, ps, ws, kv_reuse=True)
    torch.cuda.synchronize()
    return ref, got


def test_grouped_decode_matches_per_sequence(pa):
    """pa_decode_grouped on the prefix-shared batch (16 groups of 8 samples,
    2048 shared tokens = 4 partitions of 512): bit-identical to pa_decode;
    a member whose table is changed inside a shared partition gets a NaN
    row and every other row stays bit-identical."""
    sh = wl.PREFIX_SHARED
    dev = "cuda"
    plan = wl.prefix_plan()
    alloc, ids, k_pool, v_pool, order, pairs = build_shared_batch(pa, sh, plan, dev,
                                                                  sh.num_blocks)
    n_prompts, samples = plan.tail_lens.shape
    S = len(ids)
    stride = max(wl.blocks_needed(alloc.length(s), sh.block_size) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    maxlen = int(lens.max())
    ps = pa.pa_decode_default_partition(S, sh.num_kv_heads, sh.block_size, maxlen)
    groups = pa.decode_groups(tables, lens, np.arange(S) // samples, sh.block_size)[:3]
    # the 128 full prompt blocks are common; block 128 was copied on write
    assert list(groups[2]) == [2048 // sh.block_size] * n_prompts
    gen = wl.make_generator(sh.seed + 9, dev)
    q = wl.randn((S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    say(f"case grouped decode: {n_prompts} groups of {samples}, ps {ps}")
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, groups, ps, samples)
    assert torch.isfinite(ref).all()
    assert torch.equal(got, ref)
    # and every member of every group against the fp64 oracle
    want = oracle_decode_all(q, k_pool, v_pool, tables, lens, sh.block_size, sh.scale,
                             pa.K_AXES, pa.V_AXES)
    err = float(np.abs(got.double().cpu().numpy() - want).max())
    say(f"  grouped: all {S} rows max err {err:.3e}")
    assert err <= TOL

    # member 3 of group 0 points one shared-partition entry at another block
    bad = tables.copy()
    bad[3, 5] = order[alloc.stats()["num_used"]]  # a block nobody holds
    ref2, got2 = _decode_pair(pa, sh, q, k_pool, v_pool, bad, lens, groups, ps, samples)
    assert torch.isnan(got2[3]).all()
    keep = torch.ones(S, dtype=torch.bool, device=dev)
    keep[3] = False
    assert torch.equal(got2[keep], ref2[keep])


@pytest.mark.parametrize("fp8", [False, True])
def test_grouped_decode_at_the_rule_partition(pa, fp8):
    """The prefix-shared batch at the partition size pa_decode_grouped_partition
    picks for it (4096 tokens: every context fits one partition, so each
    member is split only at its group's 2048-token region), with the
    streaming policy, the workspace sized by pa_decode_grouped_workspace_size:
    every row against the fp64 oracle and within 1e-5 of per-sequence decode."""
    sh = wl.PREFIX_SHARED
    dev = "cuda"
    plan = wl.prefix_plan()
    alloc, ids, k_pool, v_pool, order, pairs = build_shared_batch(pa, sh, plan, dev,
                                                                  sh.num_blocks)
    n_prompts, samples = plan.tail_lens.shape
    S = len(ids)
    stride = max(wl.blocks_needed(alloc.length(s), sh.block_size) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    maxlen = int(lens.max())
    groups = pa.decode_groups(tables, lens, np.arange(S) // samples, sh.block_size)
    ps = pa.decode_grouped_partition(lens, *groups, sh.num_q_heads, sh.num_kv_heads,
                                     sh.block_size, maxlen)
    assert ps == 4096 and maxlen <= ps
    gen = wl.make_generator(sh.seed + 11, dev)
    q = wl.randn((S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    t_dev, l_dev = torch.as_tensor(tables, device=dev), torch.as_tensor(lens, device=dev)
    off, sg, shd = (torch.as_tensor(a, device=dev) for a in groups[:3])
    ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                             maxlen, ps, dev, grouped=True)
    got = torch.full((S, sh.num_q_heads, sh.head_dim), 7.0, device=dev)
    ref = torch.full_like(got, 7.0)
    say(f"case grouped decode at the rule's partition ({ps} tokens), fp8 {fp8}")
    if fp8:
        sc = wl.FP8_SCALE
        k8 = (k_pool.float() / sc).to(torch.float8_e4m3fn).view(torch.uint8)
        v8 = (v_pool.float() / sc).to(torch.float8_e4m3fn).view(torch.uint8)
        pa.pa_decode_grouped_fp8(got, q, k8, v8, t_dev, l_dev, sh.scale, sc, sc, maxlen, off, sg,
                                 shd, samples, ps, ws)
        pa.pa_decode_fp8(ref, q, k8, v8, t_dev, l_dev, sh.scale, sc, sc, maxlen, ps, ws)
        kk, vv, scales = k8, v8, (sc, sc)
    else:
        pa.pa_decode_grouped(got, q, k_pool, v_pool, t_dev, l_dev, sh.scale, maxlen, off, sg,
                             shd, samples, ps, ws)
        pa.pa_decode(ref, q, k_pool, v_pool, t_dev, l_dev, sh.scale, maxlen, ps, ws)
        kk, vv, scales = k_pool, v_pool, ()
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    diff = (got - ref).abs().max().item()
    want = oracle_decode_all(q, kk, vv, tables, lens, sh.block_size, sh.scale, pa.K_AXES,
                             pa.V_AXES, *scales)
    err = float(np.abs(got.double().cpu().numpy() - want).max())
    say(f"  all {S} rows: vs per-sequence {diff:.2e}, vs oracle {err:.3e}")
    assert diff <= 1e-5 and err <= TOL


def test_grouped_decode_chunks_caps_and_loners(pa):
    """GQA heads (4 members per wave, groups of 6 in two chunks), a group
    left ungrouped, a group whose shared count is far too large, and an
    empty group run.  The prompt's 18 common blocks (288 tokens) end on a
    partition boundary at 32-token partitions (bit-identical to pa_decode)
    and inside one at 64 (the region's last partition is partial: equal to
    pa_decode up to the merge's rounding, every row against the oracle)."""
    sh = wl.DecodeShape("grp", 18, 32, 8, 128, 16, 4096, "bf16", wl.SEED_BASE + 44)
    dev = "cuda"
    plan = wl.prefix_plan(num_prompts=3, samples=6, prompt_len=300, seed=sh.seed, max_tail=200)
    alloc, ids, k_pool, v_pool, order, pairs = build_shared_batch(pa, sh, plan, dev,
                                                                  sh.num_blocks)
    S = len(ids)
    stride = max(wl.blocks_needed(alloc.length(s), sh.block_size) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    seq_group = np.array([0] * 6 + [1] * 6 + [-1] * 6, np.int32)
    off, sg, shd, _ = pa.decode_groups(tables, lens, seq_group, sh.block_size)
    assert list(shd) == [300 // 16] * 2  # the prompt's full blocks
    gen = wl.make_generator(sh.seed + 1, dev)
    q = wl.randn((S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    say("case grouped decode: GQA chunks, loners")
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, (off, sg, shd), 32, 6)
    assert torch.isfinite(ref).all() and torch.equal(got, ref)
    want = oracle_decode_all(q, k_pool, v_pool, tables, lens, sh.block_size, sh.scale,
                             pa.K_AXES, pa.V_AXES)
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, (off, sg, shd), 64, 6)
    assert torch.isfinite(got).all() and torch.equal(got[12:], ref[12:])  # the loners
    assert (got - ref).abs().max().item() <= 1e-5
    err = float(np.abs(got.double().cpu().numpy() - want).max())
    say(f"  288 shared tokens at 64-token partitions: all rows vs oracle {err:.3e}")
    assert err <= TOL

    # group 1 claims 100 shared blocks (1600 tokens), more than any member's
    # context: no member shares, each is decoded alone and exactly
    shd_big = shd.copy()
    shd_big[1] = 100
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, (off, sg, shd_big), 32, 6)
    assert torch.equal(got[6:], ref[6:])
    # a claim of 25 blocks (400 tokens) reaches past the prompt: members whose
    # context goes past it share it through the leader's table, and their own
    # tables differ from the leader's there (NaN rows); the leader and the
    # members whose context ends inside it are exact
    shd_mid = shd.copy()
    shd_mid[1] = 25
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, (off, sg, shd_mid), 32, 6)
    assert torch.equal(got[:6], ref[:6]) and torch.equal(got[12:], ref[12:])
    assert (got[6] - ref[6]).abs().max().item() <= 1e-5
    for s in range(7, 12):
        if int(lens[s]) > 400:
            assert torch.isnan(got[s]).all(), s
        else:
            assert torch.equal(got[s], ref[s]), s

    # an empty run between two groups, and max_group_size below a group's size
    # (members past it are decoded alone): still bit-identical
    off2 = np.array([0, 6, 6, 12], np.int32)
    sg2 = np.array([0] * 6 + [2] * 6 + [-1] * 6, np.int32)
    shd2 = np.array([shd[0], 7, shd[1]], np.int32)
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, (off2, sg2, shd2), 32, 3)
    assert torch.equal(got, ref)


@pytest.mark.parametrize("g,bs,ps", [(1, 16, 64), (4, 16, 128), (8, 32, 256), (1, 128, 512)])
def test_grouped_decode_shared_region_inside_partitions(pa, g, bs, ps):
    """Prompts of random lengths: each group's shared region ends at an
    arbitrary block, mostly inside a partition (with 16-token blocks also
    inside a 32-token step).  Every row against the fp64 oracle and against
    pa_decode (the same terms merged at other split points); a member whose
    context ends exactly at the region's end is decoded alone, exactly."""
    hkv = 2
    sh = wl.DecodeShape("grp_split", 40, hkv * g, hkv, 128, bs, 2400, "bf16",
                        wl.SEED_BASE + 47 + g)
    dev = "cuda"
    rng = np.random.default_rng(sh.seed)
    n_prompts, samples = 10, 4
    plan = wl.PrefixPlan(rng.integers(bs + 1, 1500, n_prompts).astype(np.int32),
                         rng.integers(1, 300, (n_prompts, samples)).astype(np.int32))
    alloc, ids, k_pool, v_pool, order, pairs = build_shared_batch(pa, sh, plan, dev,
                                                                  sh.num_blocks)
    S = len(ids)
    stride = max(wl.blocks_needed(alloc.length(s), bs) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    groups = pa.decode_groups(tables, lens, np.arange(S) // samples, bs)
    shd = groups[2]
    assert (shd == plan.shared_lens // bs).all()
    # member 2 of prompt 0 decodes only up to the region's end
    lens = lens.copy()
    lens[2] = int(shd[0]) * bs
    groups = pa.decode_groups(tables, lens, np.arange(S) // samples, bs)
    assert (groups[2] == shd).all()
    off_ps = [(int(t) * bs) % ps for t in shd]
    say(f"case grouped split: G {g}, block {bs}, ps {ps}, region ends {off_ps} into a partition")
    assert sum(o != 0 for o in off_ps) >= n_prompts // 2
    gen = wl.make_generator(sh.seed + 1, dev)
    q = wl.randn((S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, groups[:3], ps, samples)
    assert torch.isfinite(got).all()
    assert torch.equal(got[2], ref[2])
    diff = (got - ref).abs().max().item()
    want = oracle_decode_all(q, k_pool, v_pool, tables, lens, bs, sh.scale, pa.K_AXES, pa.V_AXES)
    err = float(np.abs(got.double().cpu().numpy() - want).max())
    say(f"  all {S} rows: vs pa_decode {diff:.2e}, vs oracle {err:.3e}")
    assert diff <= 1e-5 and err <= TOL


def test_grouped_decode_fp8_matches_per_sequence(pa):
    """pa_decode_grouped_fp8 against pa_decode_fp8 on a small prefix-shared
    batch whose pools hold E4M3 codes: bit-identical."""
    sh = wl.DecodeShape("grp8", 12, 8, 2, 128, 16, 2048, "bf16", wl.SEED_BASE + 45)
    dev = "cuda"
    plan = wl.prefix_plan(num_prompts=3, samples=4, prompt_len=200, seed=sh.seed, max_tail=100)
    alloc, ids, k_pool, v_pool, order, pairs = build_shared_batch(pa, sh, plan, dev,
                                                                  sh.num_blocks)
    S = len(ids)
    stride = max(wl.blocks_needed(alloc.length(s), sh.block_size) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    sc = wl.FP8_SCALE
    k8 = (k_pool.float() / sc).to(torch.float8_e4m3fn).view(torch.uint8)
    v8 = (v_pool.float() / sc).to(torch.float8_e4m3fn).view(torch.uint8)
    ps = 64
    off, sg, shd, _ = pa.decode_groups(tables, lens, np.arange(S) // 4, sh.block_size)
    assert (shd == 12).all()  # 200 tokens: 12 common full blocks = 3 partitions of 64
    gen = wl.make_generator(sh.seed + 2, dev)
    q = wl.randn((S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    maxlen = int(lens.max())
    t_dev, l_dev = torch.as_tensor(tables, device=dev), torch.as_tensor(lens, device=dev)
    ws = pa.decode_workspace(S, sh.num_q_heads, sh.num_kv_heads, sh.head_dim, sh.block_size,
                             maxlen, ps, dev, grouped=True)
    ref = torch.full((S, sh.num_q_heads, sh.head_dim), 7.0, device=dev)
    got = torch.full_like(ref, 7.0)
    say("case grouped decode fp8")
    pa.pa_decode_fp8(ref, q, k8, v8, t_dev, l_dev, sh.scale, sc, sc, maxlen, ps, ws)
    pa.pa_decode_grouped_fp8(got, q, k8, v8, t_dev, l_dev, sh.scale, sc, sc, maxlen,
                             *(torch.as_tensor(a, device=dev) for a in (off, sg, shd)), 4, ps,
                             ws)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all() and torch.equal(got, ref)


@pytest.mark.parametrize("bad", ["runs_past_the_batch", "ids_out_of_range", "negative_shared",
                                 "decreasing_offsets"])
def test_grouped_decode_malformed_groups_decode_alone(pa, bad):
    """Group arrays that name no valid group leave every sequence to the
    per-sequence path: the output equals pa_decode bit for bit."""
    sh = wl.DecodeShape("grpbad", 12, 8, 8, 128, 16, 2048, "bf16", wl.SEED_BASE + 46)
    dev = "cuda"
    plan = wl.prefix_plan(num_prompts=3, samples=4, prompt_len=200, seed=sh.seed, max_tail=100)
    alloc, ids, k_pool, v_pool, order, pairs = build_shared_batch(pa, sh, plan, dev,
                                                                  sh.num_blocks)
    S = len(ids)
    stride = max(wl.blocks_needed(alloc.length(s), sh.block_size) for s in ids) + 1
    tables, lens = alloc.batch_tables(ids, stride, sh.num_blocks - 1)
    ps = 64
    off = np.array([0, 4, 8, 12], np.int32)
    sg = (np.arange(S) // 4).astype(np.int32)
    shd = np.full(3, 3, np.int32)
    if bad == "runs_past_the_batch":
        off = off + S
    elif bad == "ids_out_of_range":
        sg = sg + 3
    elif bad == "negative_shared":
        shd = shd - 6
    else:
        off = off[::-1].copy()
    gen = wl.make_generator(sh.seed + 3, dev)
    q = wl.randn((S, sh.num_q_heads, sh.head_dim), torch.bfloat16, gen, dev)
    say(f"case grouped decode, malformed groups: {bad}")
    ref, got = _decode_pair(pa, sh, q, k_pool, v_pool, tables, lens, (off, sg, shd), ps, 4)
    assert torch.isfinite(ref).all() and torch.equal(got, ref)


def test_prefix_cache_host_tier_round_trip(pa):
    """Released prompt blocks are offloaded to the host tier (pa_swap_blocks
    device -> host with the allocator's pairs), their device blocks are
    reused and overwritten by another request, then a new request with the
    same prompt reloads them (pa_seq_create_prefix_ex, host -> device
    copies) and decodes bit for bit like the same prompt written afresh; its
    rows match the fp64 oracle."""
    sh = wl.DecodeShape("host_tier", 2, 8, 4, 64, 16, 96, "bf16", 78)
    dev = "cuda"
    hkv, d, bs, nb, nh = sh.num_kv_heads, sh.head_dim, sh.block_size, sh.num_blocks, 48
    gen = wl.make_generator(sh.seed, dev)
    rng = np.random.default_rng(sh.seed)
    prompt = rng.integers(0, 1000, 40 * bs + 7).astype(np.int32)
    kp = wl.randn((len(prompt), hkv, d), torch.bfloat16, gen, dev)
    vp = wl.randn((len(prompt), hkv, d), torch.bfloat16, gen, dev)
    kshape, vshape = pa.kv_cache_shapes(nb, hkv, bs, d)
    k_pool = torch.full(kshape, float("nan"), dtype=torch.bfloat16, device=dev)
    v_pool = torch.full(vshape, float("nan"), dtype=torch.bfloat16, device=dev)
    hk, hv = pa.kv_cache_shapes(nh, hkv, bs, d)
    k_host = torch.empty(hk, dtype=torch.bfloat16, pin_memory=True)
    v_host = torch.empty(hv, dtype=torch.bfloat16, pin_memory=True)
    alloc = pa.Allocator(nb, bs, free_order=rng.permutation(nb))
    alloc.set_swap_space(nh)

    def write(seq, lo):
        slots, pairs = alloc.append_tokens(seq, prompt[lo:])
        assert len(pairs) == 0
        pa.pa_cache_write(kp[lo:].contiguous(), vp[lo:].contiguous(), k_pool, v_pool,
                          torch.as_tensor(slots, device=dev))

    assert alloc.create_prefix(1, prompt, len(prompt) - 1) == 0
    write(1, 0)
    alloc.free(1)
    out_pairs = alloc.offload(64)
    assert len(out_pairs) == len(prompt) // bs  # every full block of the prompt
    pa.pa_swap_blocks(k_pool, v_pool, k_host, v_host, torch.as_tensor(out_pairs, device=dev))
    # another request takes the freed blocks and overwrites them
    alloc.create(2)
    slots, _ = alloc.append(2, nb * bs - 8 * bs)
    junk = torch.full((len(slots), hkv, d), 3.0, dtype=torch.bfloat16, device=dev)
    pa.pa_cache_write(junk, junk, k_pool, v_pool, torch.as_tensor(slots, device=dev))
    alloc.free(2)
    # the prompt again: every full block comes back from the host
    n, in_pairs = alloc.create_prefix_ex(3, prompt, len(prompt) - 1)
    assert n == len(prompt) // bs * bs and len(in_pairs) == len(prompt) // bs
    pa.pa_swap_blocks(k_host, v_host, k_pool, v_pool, torch.as_tensor(in_pairs, device=dev))
    write(3, n)
    st = alloc.host_stats()
    say(f"case prefix host tier: offloaded {st['offloaded_blocks']}, reloaded "
        f"{st['reloaded_blocks']} blocks")
    assert st["reloaded_blocks"] == len(in_pairs) and st["host_cached_blocks"] == 0
    # the same prompt written in full into a second pool
    k2 = torch.full_like(k_pool, float("nan"))
    v2 = torch.full_like(v_pool, float("nan"))
    fresh = pa.Allocator(nb, bs)
    fresh.create(3)
    fs, _ = fresh.append(3, len(prompt))
    pa.pa_cache_write(kp, vp, k2, v2, torch.as_tensor(fs, device=dev))
    q = wl.randn((1, sh.num_q_heads, d), torch.bfloat16, gen, dev)
    outs = []
    for al, kk, vv in ((alloc, k_pool, v_pool), (fresh, k2, v2)):
        t, lens = al.batch_tables([3], 48, nb - 1)
        o = torch.empty((1, sh.num_q_heads, d), device=dev)
        ws = pa.decode_workspace(1, sh.num_q_heads, hkv, d, bs, int(lens[0]), 64, dev)
        pa.pa_decode(o, q, kk, vv, torch.as_tensor(t, device=dev),
                     torch.as_tensor(lens, device=dev), sh.scale, int(lens[0]), 64, ws)
        outs.append((o, t, lens))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0][0]).all() and torch.equal(outs[0][0], outs[1][0])
    ref = oracle_decode_all(q, k_pool, v_pool, outs[0][1], outs[0][2], bs, sh.scale, pa.K_AXES,
                            pa.V_AXES)
    err = float(np.abs(outs[0][0].double().cpu().numpy() - ref).max())
    say(f"  reloaded == fresh bit for bit; oracle err {err:.3e}")
    assert err <= TOL

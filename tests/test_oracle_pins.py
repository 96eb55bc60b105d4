"""Pins for the fp64 oracle: results the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a library
attention routine (torch's scaled_dot_product_attention in float64) on
contiguous data, closed forms, exact invariants, and cited worked examples.
Sources (page title, section):
  [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1, §3.3
  [VF] 《大模型推理：vLLM大模型推理框架（附下载）》 §1.1
  [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》 code example 1, learning points
  [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §1, §2.1
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


# ---------------------------------------------------------------------------
# helpers: contiguous data, paged by chunking tokens into blocks of BS in order


def bits(x: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.to(torch.float32).contiguous().numpy()
    return x.to(torch.bfloat16).contiguous().view(torch.int16).numpy().view(np.uint16)


def page_sequences(seqs, block_size, num_blocks, rng, axes="bhrd", fill=np.nan):
    """Lay contiguous [L][H][D] arrays (float32 or uint16 bits) into a pool.

    Tokens are cut into consecutive chunks of ``block_size`` (the last chunk
    padded with ``fill``), and chunk j of sequence s goes to physical block
    tables[s][j]; physical ids come from a random permutation.  Returns
    (pool with the given axes, tables)."""
    h, d = seqs[0].shape[1:]
    dt = seqs[0].dtype
    counts = [-(-x.shape[0] // block_size) for x in seqs]
    perm = rng.permutation(num_blocks)
    assert sum(counts) <= num_blocks
    pad = np.array(np.nan, dtype=np.float32)
    if dt == np.uint16:
        pad = np.array([0x7FC0], dtype=np.uint16)[0]
    pool = np.full((num_blocks, h, block_size, d), pad, dtype=dt)
    tables = np.zeros((len(seqs), max(counts + [1])), dtype=np.int32)
    off = 0
    for s, x in enumerate(seqs):
        n = counts[s]
        padded = np.full((n * block_size, h, d), pad, dtype=dt)
        padded[: x.shape[0]] = x
        chunks = padded.reshape(n, block_size, h, d).transpose(0, 2, 1, 3)  # [n][h][r][d]
        ids = perm[off:off + n]
        pool[ids] = chunks
        tables[s, :n] = ids
        off += n
    order = ["bhrd".index(a) for a in axes]
    return np.ascontiguousarray(pool.transpose(order)), tables


def sdpa(q, K, V, scale, mask=None):
    """Library attention in float64: q [Hq][Lq][D], K/V [Hq][L][D]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale).numpy()


def random_decode(rng, lengths, hq, hkv, d, bs, dtype, axes=("bhrd", "bhrd"), extra_blocks=3):
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    kc = [bits(torch.randn(L, hkv, d, generator=g), dtype) for L in lengths]
    vc = [bits(torch.randn(L, hkv, d, generator=g), dtype) for L in lengths]
    q = bits(torch.randn(len(lengths), hq, d, generator=g), dtype)
    nb = sum(-(-L // bs) for L in lengths) + extra_blocks
    seed = int(rng.integers(1 << 30))
    kp, tables = page_sequences(kc, bs, nb, np.random.default_rng(seed), axes[0])
    vp, tables2 = page_sequences(vc, bs, nb, np.random.default_rng(seed), axes[1])
    assert (tables == tables2).all()
    return q, kc, vc, kp, vp, tables


# ---------------------------------------------------------------------------
# attention against a library routine on contiguous data


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
@pytest.mark.parametrize("bs,axes", [(4, ("bhrd", "bhrd")), (16, ("bhrd", "bhdr")),
                                     (8, ("hbdr", "rdbh"))])
def test_decode_matches_library_attention(dtype, hq, hkv, bs, axes):
    rng = np.random.default_rng(hash((dtype, hq, hkv, bs)) % (1 << 32))
    lengths = [1, 5, bs, bs + 1, 3 * bs - 1, 37]
    d = 16
    q, kc, vc, kp, vp, tables = random_decode(rng, lengths, hq, hkv, d, bs, dtype, axes)
    scale = 1.0 / math.sqrt(d)
    out = oracle.decode(q, kp, vp, tables, lengths, scale, axes[0], axes[1])
    g = hq // hkv
    qd = oracle.widen(q)
    for s, L in enumerate(lengths):
        K = np.repeat(oracle.widen(kc[s]).transpose(1, 0, 2), g, axis=0)  # [Hq][L][D]
        V = np.repeat(oracle.widen(vc[s]).transpose(1, 0, 2), g, axis=0)
        ref = sdpa(qd[s][:, None, :], K, V, scale)[:, 0, :]
        assert np.abs(out[s] - ref).max() <= 1e-12


def test_zero_length_row_is_zero():
    rng = np.random.default_rng(7)
    q, kc, vc, kp, vp, tables = random_decode(rng, [3, 9], 2, 2, 8, 4, "f32")
    out = oracle.decode(q, kp, vp, tables, [0, 9], 0.5)
    assert (out[0] == 0).all()
    assert np.isfinite(out).all()


# ---------------------------------------------------------------------------
# exact invariants


def test_block_permutation_invariance():
    """Where the blocks sit in the pool must not change the result ([VE] §3.1:
    blocks need not be contiguous)."""
    rng = np.random.default_rng(11)
    lengths = [33, 70, 16]
    d, bs = 32, 16
    g = torch.Generator().manual_seed(5)
    kc = [bits(torch.randn(L, 2, d, generator=g), "bf16") for L in lengths]
    vc = [bits(torch.randn(L, 2, d, generator=g), "bf16") for L in lengths]
    q = bits(torch.randn(3, 4, d, generator=g), "bf16")
    outs = []
    for seed in (1, 2, 3):
        kp, t = page_sequences(kc, bs, 40, np.random.default_rng(seed))
        vp, _ = page_sequences(vc, bs, 40, np.random.default_rng(seed))
        outs.append(oracle.decode(q, kp, vp, t, lengths, 0.3))
    assert (outs[0] == outs[1]).all() and (outs[0] == outs[2]).all()


def test_length_one_returns_v_exactly():
    """One key: the single weight is exp(0)/exp(0) = 1, so out = V_0."""
    rng = np.random.default_rng(3)
    q, kc, vc, kp, vp, tables = random_decode(rng, [1, 1, 1], 4, 2, 16, 16, "bf16")
    out = oracle.decode(q, kp, vp, tables, [1, 1, 1], 0.25)
    for s in range(3):
        v0 = oracle.widen(vc[s])[0]  # [Hkv][D]
        assert (out[s] == np.repeat(v0, 2, axis=0)).all()


def test_softmax_rows_sum_to_one():
    """With every V element equal to 1 the output is the row sum of the
    softmax weights, which must be 1."""
    rng = np.random.default_rng(4)
    lengths = [1, 7, 50, 129]
    q, kc, vc, kp, vp, tables = random_decode(rng, lengths, 4, 4, 16, 16, "f32")
    ones = [np.ones_like(v) for v in vc]
    vp1, t1 = page_sequences(ones, 16, vp.shape[0], np.random.default_rng(0))
    kp1, _ = page_sequences(kc, 16, vp.shape[0], np.random.default_rng(0))
    out = oracle.decode(q, kp1, vp1, t1, lengths, 3.0)
    assert np.abs(out - 1.0).max() <= 1e-12


def test_scale_zero_gives_mean_of_v():
    rng = np.random.default_rng(5)
    lengths = [9, 40]
    q, kc, vc, kp, vp, tables = random_decode(rng, lengths, 2, 2, 8, 4, "f32")
    out = oracle.decode(q, kp, vp, tables, lengths, 0.0)
    for s in range(2):
        mean = oracle.widen(vc[s]).mean(axis=0)
        assert np.abs(out[s] - mean).max() <= 1e-12


def test_identical_keys_give_mean_and_identical_values_give_value():
    rng = np.random.default_rng(6)
    L, h, d, bs = 23, 2, 8, 4
    g = torch.Generator().manual_seed(9)
    krow = torch.randn(1, h, d, generator=g)
    kc = [bits(krow.repeat(L, 1, 1), "f32")]
    vc = [bits(torch.randn(L, h, d, generator=g), "f32")]
    q = bits(torch.randn(1, h, d, generator=g), "f32")
    kp, t = page_sequences(kc, bs, 10, np.random.default_rng(1))
    vp, _ = page_sequences(vc, bs, 10, np.random.default_rng(1))
    out = oracle.decode(q, kp, vp, t, [L], 0.7)
    assert np.abs(out[0] - oracle.widen(vc[0]).mean(axis=0)).max() <= 1e-12
    vrow = torch.randn(1, h, d, generator=g)
    vc2 = [bits(vrow.repeat(L, 1, 1), "f32")]
    kc2 = [bits(torch.randn(L, h, d, generator=g), "f32")]
    kp2, t2 = page_sequences(kc2, bs, 10, np.random.default_rng(2))
    vp2, _ = page_sequences(vc2, bs, 10, np.random.default_rng(2))
    out2 = oracle.decode(q, kp2, vp2, t2, [L], 0.7)
    assert np.abs(out2[0] - oracle.widen(vc2[0])[0]).max() <= 1e-14


def test_gqa_equals_mha_with_replicated_kv_heads():
    rng = np.random.default_rng(8)
    lengths = [17, 33]
    hq, hkv, d, bs = 8, 2, 16, 8
    q, kc, vc, kp, vp, tables = random_decode(rng, lengths, hq, hkv, d, bs, "bf16")
    out = oracle.decode(q, kp, vp, tables, lengths, 0.25)
    g = hq // hkv
    kr = [np.repeat(k, g, axis=1) for k in kc]
    vr = [np.repeat(v, g, axis=1) for v in vc]
    kp2, t2 = page_sequences(kr, bs, kp.shape[0], np.random.default_rng(3))
    vp2, _ = page_sequences(vr, bs, kp.shape[0], np.random.default_rng(3))
    out2 = oracle.decode(q, kp2, vp2, t2, lengths, 0.25)
    assert (out == out2).all()


def test_shared_blocks_equal_duplicated_storage():
    """Two sequences whose tables name the same physical prefix blocks give the
    same result as two private copies of that prefix ([VE] §3.1, KV sharing;
    [NV] learning points: shared blocks are read-only)."""
    bs, h, d = 4, 2, 8
    g = torch.Generator().manual_seed(12)
    prefix_k = bits(torch.randn(8, h, d, generator=g), "f32")  # two full blocks
    prefix_v = bits(torch.randn(8, h, d, generator=g), "f32")
    tails_k = [bits(torch.randn(n, h, d, generator=g), "f32") for n in (3, 6)]
    tails_v = [bits(torch.randn(n, h, d, generator=g), "f32") for n in (3, 6)]
    q = bits(torch.randn(2, h, d, generator=g), "f32")
    lengths = [11, 14]
    # duplicated storage: each sequence has its own copy of the prefix
    kp, t = page_sequences([np.concatenate([prefix_k, tk]) for tk in tails_k], bs, 12,
                           np.random.default_rng(4))
    vp, _ = page_sequences([np.concatenate([prefix_v, tv]) for tv in tails_v], bs, 12,
                           np.random.default_rng(4))
    dup = oracle.decode(q, kp, vp, t, lengths, 0.5)
    # shared storage: sequence 1's first two table entries point at sequence 0's blocks
    t_shared = t.copy()
    t_shared[1, :2] = t[0, :2]
    kp[t[1, :2]] = np.nan
    vp[t[1, :2]] = np.nan
    shared = oracle.decode(q, kp, vp, t_shared, lengths, 0.5)
    assert (dup == shared).all()


# ---------------------------------------------------------------------------
# prefill


def _prefill_case(rng, ctx, qlen, hq, hkv, d, bs, dtype="bf16"):
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    kc = [bits(torch.randn(c, hkv, d, generator=g), dtype) for c in ctx]
    vc = [bits(torch.randn(c, hkv, d, generator=g), dtype) for c in ctx]
    cu = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q = bits(torch.randn(int(cu[-1]), hq, d, generator=g), dtype)
    nb = sum(-(-c // bs) for c in ctx) + 2
    kp, t = page_sequences(kc, bs, nb, np.random.default_rng(1))
    vp, _ = page_sequences(vc, bs, nb, np.random.default_rng(1))
    return q, kc, vc, kp, vp, t, cu


def test_prefill_matches_library_causal_attention():
    rng = np.random.default_rng(21)
    ctx, qlen = [20, 9, 33], [7, 9, 1]
    hq, hkv, d, bs = 4, 2, 16, 8
    q, kc, vc, kp, vp, t, cu = _prefill_case(rng, ctx, qlen, hq, hkv, d, bs)
    scale = 0.25
    out = oracle.prefill(q, kp, vp, t, cu, ctx, scale)
    qd = oracle.widen(q)
    g = hq // hkv
    for r, (c, n) in enumerate(zip(ctx, qlen)):
        K = np.repeat(oracle.widen(kc[r]).transpose(1, 0, 2), g, axis=0)
        V = np.repeat(oracle.widen(vc[r]).transpose(1, 0, 2), g, axis=0)
        rows = qd[cu[r]:cu[r + 1]].transpose(1, 0, 2)  # [Hq][n][D]
        pos = c - n + np.arange(n)
        mask = np.arange(c)[None, :] <= pos[:, None]  # [n][c], bool: True = attend
        ref = sdpa(rows, K, V, scale, mask)
        assert np.abs(out[cu[r]:cu[r + 1]] - ref.transpose(1, 0, 2)).max() <= 1e-12


def test_prefill_last_row_and_single_row_equal_decode():
    rng = np.random.default_rng(22)
    ctx, qlen = [26, 13], [6, 1]
    hq, hkv, d, bs = 4, 4, 8, 4
    q, kc, vc, kp, vp, t, cu = _prefill_case(rng, ctx, qlen, hq, hkv, d, bs)
    out = oracle.prefill(q, kp, vp, t, cu, ctx, 0.3)
    last_rows = q[[cu[1] - 1, cu[2] - 1]]
    dec = oracle.decode(last_rows, kp, vp, t, ctx, 0.3)
    assert (out[cu[1] - 1] == dec[0]).all()
    assert (out[cu[2] - 1] == dec[1]).all()
    # an inner row at position p equals decode over p + 1 keys
    p_row = cu[0] + 2
    pos = ctx[0] - qlen[0] + 2
    dec2 = oracle.decode(q[[p_row]], kp, vp, t[[0]], [pos + 1], 0.3)
    assert (out[p_row] == dec2[0]).all()


# ---------------------------------------------------------------------------
# cache write and block copy (bit-exact by definition)


@pytest.mark.parametrize("axes", [("bhrd", "bhdr"), ("bhrd", "bhrd")])
def test_cache_write_then_unpage_gives_tokens_back(axes):
    """Writing tokens at pos // BS, pos % BS of their table and reading the
    table back returns them bit for bit ([VF] §1.1); untouched bytes keep
    their poison."""
    bs, h, d, nb = 4, 3, 8, 16
    rng = np.random.default_rng(31)
    perm = rng.permutation(nb)
    lengths = [6, 9]
    tables = [perm[0:2], perm[2:5]]
    g = torch.Generator().manual_seed(3)
    toks = [bits(torch.randn(L, h, d, generator=g), "bf16") for L in lengths]
    vtoks = [bits(torch.randn(L, h, d, generator=g), "bf16") for L in lengths]
    dims = {"b": nb, "h": h, "r": bs, "d": d}
    kp = np.full([dims[a] for a in axes[0]], 0x7FC0, dtype=np.uint16)
    vp = np.full([dims[a] for a in axes[1]], 0x7FC0, dtype=np.uint16)
    for s, L in enumerate(lengths):
        slots = np.array([tables[s][p // bs] * bs + p % bs for p in range(L)], dtype=np.int64)
        oracle.cache_write(toks[s], vtoks[s], kp, vp, slots, axes[0], axes[1])
    for s, L in enumerate(lengths):
        for hh in range(h):
            k = oracle.unpage(kp, axes[0], tables[s], L, hh)
            v = oracle.unpage(vp, axes[1], tables[s], L, hh)
            assert (k == oracle.widen(toks[s][:, hh])).all()
            assert (v == oracle.widen(vtoks[s][:, hh])).all()
    # exactly sum(lengths) * h * d elements changed, in each pool
    assert (kp != 0x7FC0).sum() == sum(lengths) * h * d
    assert (vp != 0x7FC0).sum() == sum(lengths) * h * d
    # a negative slot writes nothing
    before = kp.copy()
    oracle.cache_write(toks[0][:1], vtoks[0][:1], kp, vp, np.array([-1]), axes[0], axes[1])
    assert (before == kp).all()


def test_copy_blocks_copies_whole_blocks():
    bs, h, d, nb = 4, 2, 8, 6
    rng = np.random.default_rng(41)
    kp = rng.standard_normal((nb, h, bs, d)).astype(np.float32)
    vp = rng.standard_normal((nb, h, d, bs)).astype(np.float32)
    k0, v0 = kp.copy(), vp.copy()
    oracle.copy_blocks(kp, vp, np.array([[1, 4], [2, 0]]), "bhrd", "bhdr")
    assert (kp[4] == k0[1]).all() and (kp[0] == k0[2]).all()
    assert (vp[4] == v0[1]).all() and (vp[0] == v0[2]).all()
    for b in (1, 2, 3, 5):
        assert (kp[b] == k0[b]).all() and (vp[b] == v0[b]).all()


def test_swap_blocks_moves_whole_blocks_between_pools():
    # [NV] best practice 5 / [VI] §2.1: blocks leave for a host pool and come
    # back; every other block of either pool stays as it was.
    bs, h, d = 4, 2, 8
    rng = np.random.default_rng(43)
    kd = rng.standard_normal((6, h, bs, d)).astype(np.float32)
    vd = rng.standard_normal((6, h, d, bs)).astype(np.float32)
    kh = rng.standard_normal((3, h, bs, d)).astype(np.float32)
    vh = rng.standard_normal((3, h, d, bs)).astype(np.float32)
    kd0, vd0, kh0, vh0 = kd.copy(), vd.copy(), kh.copy(), vh.copy()
    out = np.array([[5, 2], [1, 0]])
    oracle.swap_blocks(kd, vd, kh, vh, out, "bhrd", "bhdr")
    assert (kh[2] == kd0[5]).all() and (kh[0] == kd0[1]).all() and (kh[1] == kh0[1]).all()
    assert (vh[2] == vd0[5]).all() and (vh[0] == vd0[1]).all() and (vh[1] == vh0[1]).all()
    assert (kd == kd0).all() and (vd == vd0).all()
    kd[[5, 1]] = 0.0
    vd[[5, 1]] = 0.0
    oracle.swap_blocks(kh, vh, kd, vd, np.array([[2, 3], [0, 4]]), "bhrd", "bhdr")
    assert (kd[3] == kd0[5]).all() and (kd[4] == kd0[1]).all()
    assert (vd[3] == vd0[5]).all() and (vd[4] == vd0[1]).all()
    for b in (0, 2):
        assert (kd[b] == kd0[b]).all() and (vd[b] == vd0[b]).all()


def test_widen_is_exact():
    x = np.array([1.0, -2.5, 3.0e-39, np.inf, 65504.0, 1.0e38], dtype=np.float32)
    b = torch.from_numpy(x).to(torch.bfloat16)
    bbits = b.view(torch.int16).numpy().view(np.uint16)
    assert (oracle.widen(bbits) == b.to(torch.float64).numpy()).all()
    assert (oracle.widen(x) == x.astype(np.float64)).all()


# -- fp8 (OCP E4M3) codec and the quantized cache -------------------------------
# The pages give no fp8 format or scale; the reading here (OCP E4M3, one scale per
# cache, values beyond 448 saturate) is pinned against torch's float8_e4m3fn,
# which follows the same OCP definition.

def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all() and nan.sum() == 2  # 0x7F and 0xFF
    assert (ours[~nan] == ref[~nan]).all()
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_in_range_with_ties():
    finite = np.arange(0, 0x7F, dtype=np.uint8)
    vals = oracle.e4m3_decode(finite)
    mids = (vals[:-1] + vals[1:]) / 2  # every tie between neighbouring codes
    rng = np.random.default_rng(7)
    rand = rng.uniform(-460, 460, 4000)
    small = rng.uniform(-0.02, 0.02, 2000)
    x = np.concatenate([vals, -vals, mids, -mids, rand, small]).astype(np.float32)
    x = x[np.abs(x) < 464]  # torch gives NaN past 464; this oracle saturates there
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all()


def test_e4m3_encode_round_trip_saturation_and_nan():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert (oracle.e4m3_encode(oracle.e4m3_decode(codes).astype(np.float32)) == codes).all()
    big = np.array([464.0, 470.0, 1e9, np.inf, -500.0, -np.inf], dtype=np.float32)
    assert list(oracle.e4m3_encode(big)) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert oracle.e4m3_encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F
    # monotone: a larger value never gets a smaller magnitude code
    x = np.sort(np.random.default_rng(3).uniform(0, 450, 3000)).astype(np.float32)
    v = oracle.e4m3_decode(oracle.e4m3_encode(x))
    assert (np.diff(v) >= 0).all()


def test_cache_write_fp8_quantizes_each_element_by_its_cache_scale():
    bs, h, d, nb = 4, 2, 8, 3
    rng = np.random.default_rng(5)
    k_new = (rng.standard_normal((5, h, d)) * 3).astype(np.float32)
    v_new = (rng.standard_normal((5, h, d)) * 3).astype(np.float32)
    kp = np.full((nb, h, bs, d), 0xAA, dtype=np.uint8)
    vp = np.full((nb, h, d, bs), 0xAA, dtype=np.uint8)
    slots = np.array([0, 5, 11, -1, 6])
    ks, vs = np.float32(0.05), np.float32(0.0625)
    oracle.cache_write_fp8(k_new, v_new, kp, vp, slots, ks, vs, "bhrd", "bhdr")
    for t, slot in enumerate(slots):
        if slot < 0:
            continue
        b, r = slot // bs, slot % bs
        want_k = torch.from_numpy(k_new[t] / ks).to(torch.float8_e4m3fn).view(torch.uint8)
        want_v = torch.from_numpy(v_new[t] / vs).to(torch.float8_e4m3fn).view(torch.uint8)
        assert (kp[b, :, r, :] == want_k.numpy()).all()
        assert (vp[b, :, :, r] == want_v.numpy()).all()
    assert (kp[0, :, 2] == 0xAA).all()  # slot 2 untouched; the -1 slot wrote nothing


def test_decode_on_fp8_pools_uses_scaled_values():
    # an fp8 pool decodes exactly like an fp32 pool holding code value * scale
    bs, h, d = 4, 2, 8
    rng = np.random.default_rng(9)
    codes_k = rng.integers(0, 256, (4, h, bs, d)).astype(np.uint8)
    codes_v = rng.integers(0, 256, (4, h, d, bs)).astype(np.uint8)
    for c in (codes_k, codes_v):
        c[(c & 0x7F) == 0x7F] = 0x10  # no NaN codes
    ks, vs = 0.03125, 0.75  # products with E4M3 values stay exact in fp32
    fk = (oracle.e4m3_decode(codes_k) * ks).astype(np.float32)
    fv = (oracle.e4m3_decode(codes_v) * vs).astype(np.float32)
    q = rng.standard_normal((2, 4, d)).astype(np.float32)
    tables = np.array([[2, 0, 3], [1, 3, 0]], dtype=np.int32)
    lens = np.array([11, 6], dtype=np.int32)
    a = oracle.decode(q, codes_k, codes_v, tables, lens, 0.35, "bhrd", "bhdr", ks, vs)
    b = oracle.decode(q, fk, fv, tables, lens, 0.35, "bhrd", "bhdr")
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_prefill_on_fp8_pools_uses_scaled_values():
    bs, h, d = 4, 2, 8
    rng = np.random.default_rng(12)
    codes_k = rng.integers(0, 256, (5, h, bs, d)).astype(np.uint8)
    codes_v = rng.integers(0, 256, (5, h, d, bs)).astype(np.uint8)
    for c in (codes_k, codes_v):
        c[(c & 0x7F) == 0x7F] = 0x21
    ks, vs = 0.015625, 1.5  # exact products with E4M3 values in fp32
    fk = (oracle.e4m3_decode(codes_k) * ks).astype(np.float32)
    fv = (oracle.e4m3_decode(codes_v) * vs).astype(np.float32)
    q = rng.standard_normal((5, 4, d)).astype(np.float32)
    tables = np.array([[2, 0, 3, 1], [4, 1, 0, 2]], dtype=np.int32)
    ctx = np.array([13, 7], dtype=np.int32)
    cu = np.array([0, 3, 5], dtype=np.int32)
    a = oracle.prefill(q, codes_k, codes_v, tables, cu, ctx, 0.3, "bhrd", "bhdr", ks, vs)
    b = oracle.prefill(q, fk, fv, tables, cu, ctx, 0.3, "bhrd", "bhdr")
    assert np.allclose(a, b, rtol=0, atol=1e-12)

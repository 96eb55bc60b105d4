"""pa_decode_noalloc (split-K partials in the library's own device scratch,
for callers that cannot allocate) against pa_decode_ex with a caller
workspace: the same kernels and partition sizes, so the outputs must match
bit for bit, and both stay within the attention bar against the fp64
oracle.  Two calls in a row, the second on a smaller batch, so the second
reads a scratch the first left full; then a batch too large for the
scratch, which must be refused with nothing enqueued."""
import sys

import numpy as np
import pytest
import torch

import workloads as wl
from paged_helpers import oracle_decode_all

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


def case_of(pa, lengths, hq, hkv, seed):
    sh = wl.DecodeShape("noalloc", len(lengths), hq, hkv, 128, 16, 0, "bf16", seed)
    need = sum(wl.blocks_needed(L, 16) for L in lengths) + 8
    return wl.make_decode_case(sh, "cuda", pa.K_AXES, pa.V_AXES, lengths=lengths,
                               num_blocks=need)


def both(pa, case, ps):
    sh = case.shape
    dev = "cuda"
    lens = case.lengths
    maxlen = int(max(lens))
    t_dev = torch.as_tensor(case.tables, dtype=torch.int32, device=dev)
    l_dev = torch.as_tensor(lens, dtype=torch.int32, device=dev)
    ref = torch.full((len(lens), sh.num_q_heads, sh.head_dim), 7.0, device=dev)
    ws = pa.decode_workspace(len(lens), sh.num_q_heads, sh.num_kv_heads, sh.head_dim,
                             sh.block_size, maxlen, ps, dev)
    pa.pa_decode(ref, case.q, case.k_pool, case.v_pool, t_dev, l_dev, sh.scale, maxlen, ps, ws)
    got = torch.full_like(ref, 7.0)
    pa.pa_decode_noalloc(got, case.q, case.k_pool, case.v_pool, t_dev, l_dev, sh.scale, maxlen,
                         ps)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_workspace_decode_twice(pa):
    rng = np.random.default_rng(0x417)
    # call 1: 96 sequences up to 4096 tokens, GQA 32/8, 512-token partitions
    # (96 x 32 x 8 partitions of partials: 12.8 MB of the scratch)
    lens1 = [int(x) for x in rng.integers(1, 4097, size=96)]
    lens1[:3] = [4096, 1, 513]
    c1 = case_of(pa, lens1, 32, 8, 11)
    say(f"case noalloc call 1: {len(lens1)} seqs, max {max(lens1)}")
    ref1, got1 = both(pa, c1, 512)
    assert torch.equal(ref1, got1)
    err1 = float(np.abs(got1.double().cpu().numpy() - oracle_decode_all(
        c1.q, c1.k_pool, c1.v_pool, c1.tables, c1.lengths, 16, c1.shape.scale, c1.k_axes,
        c1.v_axes)).max())
    say(f"  bit-identical to pa_decode_ex; oracle max err {err1:.3e}")
    assert err1 <= TOL
    # call 2: a smaller batch (MHA 8/8, 64-token partitions), reading a
    # scratch the first call left full
    lens2 = [700, 64, 65, 1000, 5]
    c2 = case_of(pa, lens2, 8, 8, 12)
    say(f"case noalloc call 2: {len(lens2)} seqs, max {max(lens2)}")
    ref2, got2 = both(pa, c2, 64)
    assert torch.equal(ref2, got2)
    err2 = float(np.abs(got2.double().cpu().numpy() - oracle_decode_all(
        c2.q, c2.k_pool, c2.v_pool, c2.tables, c2.lengths, 16, c2.shape.scale, c2.k_axes,
        c2.v_axes)).max())
    say(f"  bit-identical to pa_decode_ex; oracle max err {err2:.3e}")
    assert err2 <= TOL
    # a batch of one partition per sequence needs no scratch at all
    ref3, got3 = both(pa, c2, 1024)
    assert torch.equal(ref3, got3)


def test_noalloc_refuses_batches_beyond_its_scratch(pa):
    c = case_of(pa, [40, 17], 32, 32, 13)
    dev = "cuda"
    t_dev = torch.as_tensor(c.tables, dtype=torch.int32, device=dev)
    l_dev = torch.as_tensor(c.lengths, dtype=torch.int32, device=dev)
    out = torch.full((2, 32, 128), 7.0, device=dev)
    # max_context_len 2^20 at 512-token partitions: 2 x 32 x 2048 partials
    # of 520 bytes, 68 MB > 64 MiB
    need = pa.pa_decode_workspace_size(2, 32, 32, 128, 16, 1 << 20, 512)
    assert need > pa.PA_DECODE_NOALLOC_SCRATCH_BYTES
    say(f"case noalloc refusal: {need} bytes needed")
    with pytest.raises(pa.PAError) as e:
        pa.pa_decode_noalloc(out, c.q, c.k_pool, c.v_pool, t_dev, l_dev, c.shape.scale, 1 << 20,
                             512)
    assert e.value.status == pa.PA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out == 7.0).all()  # nothing was enqueued

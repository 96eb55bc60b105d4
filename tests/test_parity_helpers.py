"""CPU checks of the threaded oracle drivers the full-size GPU parity tests
use: splitting a batch into per-sequence (decode) or per-slice (prefill)
oracle calls on host threads must give exactly the oracle's own result on
the whole batch (the same fp64 arithmetic per row, so bit-identical)."""
import numpy as np
import torch

import oracle
import workloads as wl
from paged_helpers import host_bits, oracle_decode_all, oracle_prefill_all


def test_threaded_decode_equals_whole_batch_oracle():
    sh = wl.DecodeShape("custom", 7, 8, 2, 64, 16, 0, "bf16", 4242)
    lens = [0, 1, 17, 64, 200, 333, 5]
    case = wl.make_decode_case(sh, "cpu", "bhrd", "bhdr", lengths=lens,
                               num_blocks=sum(wl.blocks_needed(L, 16) for L in lens) + 4)
    whole = oracle.decode(host_bits(case.q), host_bits(case.k_pool), host_bits(case.v_pool),
                          case.tables, case.lengths, sh.scale, "bhrd", "bhdr")
    split = oracle_decode_all(case.q, case.k_pool, case.v_pool, case.tables, case.lengths, 16,
                              sh.scale, "bhrd", "bhdr")
    assert np.array_equal(whole, split)
    rows = [5, 1, 3]
    assert np.array_equal(whole[rows], oracle_decode_all(
        case.q, case.k_pool, case.v_pool, case.tables, case.lengths, 16, sh.scale, "bhrd",
        "bhdr", rows=rows))


def test_threaded_prefill_equals_whole_batch_oracle():
    sh = wl.PrefillShape(num_reqs=3, num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                         seed=4243)
    ctx, ql = [300, 70, 1], [100, 70, 1]
    case = wl.make_prefill_case(sh, "cpu", "bhrd", "bhdr", context_lens=ctx, q_lens=ql)
    whole = oracle.prefill(host_bits(case.q), host_bits(case.k_pool), host_bits(case.v_pool),
                           case.tables, case.cu_q_lens, case.context_lens, sh.scale, "bhrd",
                           "bhdr")
    for per_task in (1, 7, 32, 512):
        split = oracle_prefill_all(case.q, case.k_pool, case.v_pool, case.tables,
                                   case.cu_q_lens, case.context_lens, 16, sh.scale, "bhrd",
                                   "bhdr", rows_per_task=per_task)
        assert np.array_equal(whole, split), per_task

"""Pins for the allocator reference model (oracle/allocator_model.py).

Sources (page title, section):
  [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1
  [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》 code example 1
  [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §2.1
"""
import os

import numpy as np
import pytest

from oracle.allocator_model import AllocatorModel, OutOfBlocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_counts.txt")


def golden_block_counts():
    rows = []
    for line in open(GOLDEN, encoding="utf-8"):
        if line.startswith("#") or not line.strip():
            continue
        nums = line.split("|")[0].split()
        rows.append(tuple(int(x) for x in nums))
    return rows


@pytest.mark.parametrize("seq_len,block_size,blocks", golden_block_counts())
def test_printed_block_counts(seq_len, block_size, blocks):
    a = AllocatorModel(64, block_size)
    a.create(0)
    a.append(0, seq_len)
    assert len(a.tables[0]) == blocks
    assert a.stats()["num_used"] == blocks


def test_blocks_are_ceil_of_length():
    # lengths of the tiny fp32 batch before and after one appended token
    a = AllocatorModel(64, 16)
    for s, L in enumerate([17, 64, 100, 200]):
        a.create(s)
        a.append(s, L)
    assert [len(a.tables[s]) for s in range(4)] == [2, 4, 7, 13]
    for s in range(4):
        a.append(s, 1)
    assert [len(a.tables[s]) for s in range(4)] == [2, 5, 7, 13]
    assert a.stats()["num_used"] == 27


def test_out_of_blocks_is_all_or_nothing():
    """Asking for more blocks than the pool holds is an error ([NV] code example 1)
    and leaves every table, refcount and the free list as they were."""
    a = AllocatorModel(1024, 16)
    a.create(0)
    a.append(0, 1024 * 16)
    assert a.stats()["num_free"] == 0
    a.create(1)
    snap = (list(a.stack), list(a.refcount), {k: list(v) for k, v in a.tables.items()})
    with pytest.raises(OutOfBlocks):
        a.append(1, 1)
    assert snap == (list(a.stack), list(a.refcount), {k: list(v) for k, v in a.tables.items()})
    b = AllocatorModel(4, 16)
    b.create(0)
    b.append(0, 40)  # 3 blocks
    with pytest.raises(OutOfBlocks):
        b.append(0, 40)  # would need 3 more, only 1 free
    assert b.lengths[0] == 40 and len(b.tables[0]) == 3


def test_free_returns_blocks_at_once_lifo():
    """A finished sequence's blocks go back at once ([VE] §3.1) onto the free
    list that allocation pops from ([VI] §2.1)."""
    order = [5, 2, 7, 0, 1, 3, 4, 6]
    a = AllocatorModel(8, 4, free_order=order)
    a.create(0)
    a.append(0, 9)
    assert a.tables[0] == [5, 2, 7]
    a.free(0)
    assert a.stats()["num_free"] == 8
    a.create(1)
    a.append(1, 4)
    assert a.tables[1] == [5]


def test_slots_follow_block_and_offset():
    a = AllocatorModel(16, 4, free_order=list(range(15, -1, -1)))
    a.create(0)
    slots, pairs = a.append(0, 6)
    assert a.tables[0] == [15, 14]
    assert slots == [60, 61, 62, 63, 56, 57] and pairs == []


def test_fork_shares_and_cow_copies_partial_shared_block():
    a = AllocatorModel(16, 4)
    a.create(0)
    a.append(0, 6)  # blocks 0, 1; block 1 half full
    a.fork(0, 1)
    a.fork(0, 2)
    assert a.refcount[0] == 3 and a.refcount[1] == 3
    s1, p1 = a.append(1, 1)
    assert p1 == [(1, 2)] and a.tables[1] == [0, 2] and s1 == [2 * 4 + 2]
    assert a.refcount[1] == 2 and a.refcount[2] == 1
    s2, p2 = a.append(2, 1)
    assert p2 == [(1, 3)] and a.refcount[1] == 1
    s0, p0 = a.append(0, 1)  # last holder writes in place
    assert p0 == [] and s0 == [1 * 4 + 2]
    assert a.stats()["cow_copies"] == 2


def test_fork_at_block_boundary_needs_no_copy():
    a = AllocatorModel(16, 4)
    a.create(0)
    a.append(0, 8)
    a.fork(0, 1)
    _, pairs = a.append(1, 3)
    assert pairs == [] and a.tables[1][:2] == a.tables[0][:2]


def test_random_ops_conserve_references():
    rng = np.random.default_rng(0)
    a = AllocatorModel(64, 4, free_order=rng.permutation(64))
    live = []
    next_id = 0
    for _ in range(2000):
        op = rng.integers(4)
        try:
            if op == 0 or not live:
                a.create(next_id)
                live.append(next_id)
                next_id += 1
            elif op == 1:
                a.append(live[rng.integers(len(live))], int(rng.integers(0, 9)))
            elif op == 2:
                a.fork(live[rng.integers(len(live))], next_id)
                live.append(next_id)
                next_id += 1
            else:
                s = live.pop(rng.integers(len(live)))
                a.free(s)
        except OutOfBlocks:
            pass
        refs = sum(len(t) for t in a.tables.values())
        assert refs == sum(a.refcount)
        st = a.stats()
        assert st["num_free"] + st["num_used"] == 64
        assert st["num_free"] == sum(1 for r in a.refcount if r == 0)

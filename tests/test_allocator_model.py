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


# -- prefix cache -------------------------------------------------------------
# [VI] §2.1: allocation first reuses blocks shareable with the request's prefix,
# then takes free ones; cold blocks leave under an LRU policy.  [NV] practical
# advice: the prefix-cache hit rate is the metric to watch.  The expected tables
# below are worked out by hand from that reading (keys = (parent block, tokens)).

def _prompt(a, seq, tokens, max_cached=None):
    """Serve a prompt the way a scheduler would: reuse, then append the rest."""
    n = a.create_prefix(seq, tokens, len(tokens) if max_cached is None else max_cached)
    slots, pairs = a.append(seq, len(tokens) - n, tokens=tokens[n:])
    return n, slots, pairs


def test_prefix_hit_shares_full_blocks_only():
    a = AllocatorModel(16, 4)  # blocks handed out 0, 1, 2, ...
    n, slots, _ = _prompt(a, 1, list(range(10)))       # blocks 0, 1 full, 2 partial
    assert n == 0 and a.tables[1] == [0, 1, 2]
    n, slots, _ = _prompt(a, 2, list(range(9)) + [99])  # same first 8 tokens
    assert n == 8 and a.tables[2] == [0, 1, 3]
    assert slots == [12, 13]                          # positions 8, 9 in block 3
    assert a.refcount[:4] == [2, 2, 1, 1]
    assert a.prefix_stats() == {"queried_blocks": 4, "hit_blocks": 2, "cached_blocks": 2,
                                "cached_free_blocks": 0}


def test_prefix_key_covers_the_whole_prefix():
    a = AllocatorModel(16, 4)
    _prompt(a, 1, [1, 2, 3, 4, 5, 6, 7, 8])
    # same second block, different first block: no hit at all
    n, _, _ = _prompt(a, 2, [9, 9, 9, 9, 5, 6, 7, 8])
    assert n == 0 and a.tables[2] == [2, 3]


def test_max_cached_leaves_positions_to_compute():
    a = AllocatorModel(16, 4)
    _prompt(a, 1, list(range(8)))
    n, slots, _ = _prompt(a, 2, list(range(8)), max_cached=7)
    assert n == 4 and a.tables[2] == [0, 2]  # block 1's twin not re-registered
    assert slots == [8, 9, 10, 11]
    assert a.key_of.get(2) is None


def test_released_blocks_stay_cached_and_are_revived():
    a = AllocatorModel(8, 4)
    _prompt(a, 1, list(range(12)))  # blocks 0, 1, 2 registered
    a.free(1)
    assert a.stack == [7, 6, 5, 4, 3] and a.lru == [2, 1, 0]
    assert a.stats()["num_free"] == 8
    n, _, _ = _prompt(a, 2, list(range(8)) + [50, 51])
    assert n == 8 and a.tables[2] == [0, 1, 3]  # revived 0, 1; new block from the stack
    assert a.lru == [2] and a.refcount[:4] == [1, 1, 0, 1]


def test_eviction_takes_oldest_and_drops_descendants():
    a = AllocatorModel(4, 2)
    _prompt(a, 1, [1, 2, 3, 4])   # blocks 0 <- 1 (1's parent is 0)
    _prompt(a, 2, [7, 7])         # block 2
    a.free(2)                     # lru: [2]
    a.free(1)                     # lru: [2, 1, 0]
    assert a.lru == [2, 1, 0]
    _prompt(a, 3, [5, 5, 6, 6])   # needs 2 blocks: 3 from the stack, then evicts 2
    assert a.tables[3] == [3, 2] and a.lru == [1, 0]
    _prompt(a, 4, [8, 8])         # evicts 1 (child of 0): 0 keeps its key
    assert a.tables[4] == [1]
    assert (-1, (1, 2)) in a.keys and (0, (3, 4)) not in a.keys
    a.free(4)                     # block 1 ([8, 8]) queued
    n, _, _ = _prompt(a, 5, [1, 2, 3, 4])  # only the first block hits now
    assert n == 2 and a.tables[5] == [0, 1]  # 1 evicted again for the second block
    assert a.keys[(0, (3, 4))] == 1 and (-1, (8, 8)) not in a.keys


def test_evicting_a_parent_drops_its_queued_children():
    a = AllocatorModel(3, 2)
    _prompt(a, 1, [1, 1, 2, 2])   # 0 <- 1
    a.free(1)                     # pushed last entry first: lru [1, 0]
    a.lru = [0, 1]                # reorder by hand: the parent is now the oldest
    _prompt(a, 2, [9, 9])         # takes 2 from the stack
    _prompt(a, 3, [8, 8])         # evicts 0, which drops child 1's key too
    assert a.tables[3] == [0] and a.keys == {(-1, (9, 9)): 2, (-1, (8, 8)): 0}
    assert a.lru == [1] and 1 not in a.key_of


def test_plain_append_stops_the_chain():
    a = AllocatorModel(16, 4)
    a.create(1)
    a.append(1, 2)                           # no token ids
    a.append(1, 6, tokens=[1, 2, 3, 4, 5, 6])
    assert a.keys == {}
    assert _prompt(a, 2, [1, 2, 3, 4])[0] == 0


def test_fork_continues_the_chain_and_duplicates_are_not_registered():
    a = AllocatorModel(16, 4)
    _prompt(a, 1, [1, 2, 3, 4, 5, 6])        # block 0 registered, 1 partial
    a.fork(1, 2)
    a.append(1, 2, tokens=[7, 8])            # 1 fills block 1: COW? no, 2 shares it
    a.append(2, 2, tokens=[7, 8])            # the twin fills its own copy
    k = (0, (5, 6, 7, 8))
    assert a.keys[k] in a.tables[1] and a.key_of.get(a.tables[2][1]) is None
    assert not a.chain[2] and a.chain[1]


def test_random_prefix_ops_keep_invariants():
    rng = np.random.default_rng(11)
    a = AllocatorModel(24, 2)
    live, nxt = [], 0
    vocab = [[1, 2, 3, 4, 5, 6], [1, 2, 3, 4, 7, 7], [9, 9, 1, 2], [1, 2]]
    for _ in range(400):
        op = int(rng.integers(4))
        try:
            if op == 0 or not live:
                toks = list(vocab[int(rng.integers(len(vocab)))]) + [int(rng.integers(3))]
                live.append(nxt)
                nxt += 1
                _prompt(a, live[-1], toks, max_cached=len(toks) - 1)
            elif op == 1:
                sid = live[int(rng.integers(len(live)))]
                k = int(rng.integers(1, 4))
                a.append(sid, k, tokens=[int(x) for x in rng.integers(0, 3, k)])
            elif op == 2:
                a.fork(live[int(rng.integers(len(live)))], nxt)
                live.append(nxt)
                nxt += 1
            else:
                a.free(live.pop(int(rng.integers(len(live)))))
        except OutOfBlocks:
            pass
        held = [b for t in a.tables.values() for b in t]
        assert sum(a.refcount) == len(held)
        assert sorted(a.stack + a.lru + sorted(set(held))) == list(range(24))
        for key, b in a.keys.items():
            assert a.key_of[b] == key
            assert a.refcount[b] > 0 or b in a.lru
            if key[0] >= 0:
                assert key[0] in a.key_of and b in a.children[key[0]]
                # every holder of a block holds its parent
                assert a.refcount[key[0]] >= a.refcount[b]


# -- swap space ---------------------------------------------------------------
# [NV] best practice 5: preemption swaps a request's KV cache out to CPU memory
# and back in when room returns.  [VI] §2.1: cold blocks migrate to CPU memory.
# Expected tables below are worked out by hand from that reading.

def test_swap_out_and_in_round_trip():
    a = AllocatorModel(8, 4)
    a.set_swap_space(6)
    a.create(1)
    a.append(1, 10)                       # device blocks 0, 1, 2
    a.create(2)
    a.append(2, 4)                        # device block 3
    pairs = a.swap_out(1)
    assert pairs == [(0, 0), (1, 1), (2, 2)]
    assert a.tables[1] == [0, 1, 2] and 1 in a.swapped
    assert a.stack[-3:] == [2, 1, 0]      # released last entry first
    assert a.stats()["num_free"] == 7 and a.swap_stats()["num_host_free"] == 3
    a.create(3)
    a.append(3, 5)                        # takes device 0, 1 (the swapped ones)
    assert a.tables[3] == [0, 1]
    pairs = a.swap_in(1)                  # needs 3: takes 2, then 4, 5
    assert pairs == [(0, 2), (1, 4), (2, 5)]
    assert a.tables[1] == [2, 4, 5] and a.lengths[1] == 10
    assert a.host_stack == [5, 4, 3, 2, 1, 0]
    assert a.swap_stats() == {"num_host_blocks": 6, "num_host_free": 6, "swapped_seqs": 0,
                              "swap_out_blocks": 3, "swap_in_blocks": 3}


def test_swap_out_of_a_sharer_keeps_the_others():
    a = AllocatorModel(8, 4)
    a.set_swap_space(4)
    a.create(1)
    a.append(1, 6)                        # blocks 0 (full), 1 (partial)
    a.fork(1, 2)
    assert a.refcount[:2] == [2, 2]
    pairs = a.swap_out(2)
    assert pairs == [(0, 0), (1, 1)] and a.refcount[:2] == [1, 1]
    assert a.tables[1] == [0, 1]
    a.swap_in(2)
    assert a.tables[2] == [2, 3] and a.refcount[:4] == [1, 1, 1, 1]


def test_swap_failures_change_nothing():
    a = AllocatorModel(4, 2)
    a.set_swap_space(2)
    a.create(1)
    a.append(1, 6)                        # 3 blocks
    before = (list(a.stack), list(a.host_stack), dict(a.tables), set(a.swapped))
    with pytest.raises(OutOfBlocks):
        a.swap_out(1)                     # 3 host blocks needed, 2 exist
    assert (list(a.stack), list(a.host_stack), dict(a.tables), set(a.swapped)) == before
    b = AllocatorModel(4, 2)
    b.set_swap_space(4)
    b.create(1)
    b.append(1, 6)                        # 0, 1, 2
    b.swap_out(1)
    b.create(2)
    b.append(2, 4)                        # takes 0, 1
    b.create(3)
    b.append(3, 3)                        # takes 2, 3
    with pytest.raises(OutOfBlocks):
        b.swap_in(1)                      # no device block left
    assert 1 in b.swapped and b.tables[1] == [0, 1, 2]


def test_swapped_sequence_rejects_use_and_frees_host_blocks():
    a = AllocatorModel(8, 4)
    a.set_swap_space(4)
    a.create(1)
    a.append(1, 5)
    a.swap_out(1)
    with pytest.raises(ValueError):
        a.append(1, 1)
    with pytest.raises(ValueError):
        a.fork(1, 2)
    a.free(1)
    assert a.host_stack == [3, 2, 1, 0] and a.stats()["num_free"] == 8


def test_swap_out_of_cached_blocks_keeps_them_cached():
    a = AllocatorModel(8, 2)
    a.set_swap_space(4)
    a.create_prefix(1, [5, 6, 7, 8], 4)
    a.append(1, 4, tokens=[5, 6, 7, 8])   # blocks 0, 1 registered
    a.swap_out(1)
    assert a.lru == [1, 0]                # cached, queued
    assert a.create_prefix(2, [5, 6, 7, 8, 9], 4) == 4
    assert a.tables[2] == [0, 1]
    a.swap_in(1)                          # fresh private blocks
    assert a.tables[1] == [2, 3] and not a.chain[1]

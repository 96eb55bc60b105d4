"""Pins for the continuous-batching scheduler model (oracle/scheduler_model.py).

The expected plans are worked out by hand from the policy in the model's
docstring, which reads:
  [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.2 (requests join and leave the
       batch at every iteration),
  [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §1, §2.2 (prefill
       and decode in one iteration; pending queue; resources released at once),
  [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》 best practice 5 (FCFS;
       preemption by moving a request's cache to CPU memory).
"""
import numpy as np
import pytest

from oracle.allocator_model import AllocatorModel
from oracle.scheduler_model import SchedulerModel


def sched(nb=16, bs=4, seqs=4, tokens=8, chunk=4, host=0):
    a = AllocatorModel(nb, bs)
    if host:
        a.set_swap_space(host)
    return SchedulerModel(a, seqs, tokens, chunk)


def test_chunked_prefill_within_the_token_budget():
    s = sched()
    s.add(1, 10, 3)
    s.add(2, 3, 1)
    p = s.step()
    assert p.prefill == [(1, 0, 4), (2, 0, 3)] and p.decode == []
    assert p.slots == [0, 1, 2, 3, 4, 5, 6]        # blocks 0 (req 1) and 1 (req 2)
    assert s.complete(p) == [2]                      # 2's prompt done: its one token
    p = s.step()
    assert p.prefill == [(1, 4, 4)] and p.decode == []
    assert s.complete(p) == []
    p = s.step()
    assert p.prefill == [(1, 8, 2)]                  # prompt complete: token 1
    s.complete(p)
    p = s.step()
    assert p.decode == [(1, 11)] and p.prefill == []  # position 10 appended
    s.complete(p)
    assert s.reqs[1].generated == 2
    p = s.step()
    assert p.decode == [(1, 12)]
    assert s.complete(p) == [1]
    assert s.stats()["finished"] == 2 and s.a.stats()["num_free"] == 16


def test_fcfs_head_of_queue_is_not_overtaken():
    s = sched(nb=4, bs=4, tokens=64, chunk=64)
    s.add(1, 12, 1)   # 3 blocks
    s.add(2, 8, 1)    # needs 2 blocks: does not fit after 1
    s.add(3, 2, 1)    # would fit, but waits behind 2
    p = s.step()
    assert p.prefill == [(1, 0, 12)] and list(s.waiting) == [2, 3]
    s.complete(p)     # 1 finishes at once (max_new 1) and frees its blocks
    p = s.step()
    assert p.prefill == [(2, 0, 8), (3, 0, 2)]


def test_max_num_seqs_caps_the_running_set():
    s = sched(seqs=2, tokens=64, chunk=64)
    for r in range(4):
        s.add(r, 2, 5)
    p = s.step()
    assert [x[0] for x in p.prefill] == [0, 1] and list(s.waiting) == [2, 3]


def test_decode_shortage_preempts_the_newest_by_recompute():
    # 3 blocks of 4: two requests of 6 positions hold 2 + 2 > 3 ... use 4 blocks
    s = sched(nb=4, bs=4, tokens=64, chunk=64)
    s.add(1, 8, 4)    # 2 full blocks
    s.add(2, 8, 4)    # 2 full blocks: the pool is full
    p = s.step()
    assert p.prefill == [(1, 0, 8), (2, 0, 8)]
    s.complete(p)
    p = s.step()      # both need a new block for position 8: preempt 2 (newest)
    assert p.preempted == [2] and p.decode == [(1, 9)] and list(s.waiting) == [2]
    assert s.reqs[2].done == 0 and s.stats()["recompute_preemptions"] == 1
    # 2 comes back as a new admission once blocks are free: not in this step
    # (budget 63, but 2 needs 2 blocks and 1 free)
    assert p.prefill == []


def test_decode_shortage_preempts_by_swap_and_resumes():
    s = sched(nb=4, bs=4, tokens=64, chunk=64, host=8)
    s.add(1, 8, 2)
    s.add(2, 8, 3)
    p = s.step()
    s.complete(p)
    p = s.step()
    assert p.swap_out == [(2, 0), (3, 1)] and s.swapped == [2]   # 2's blocks 2, 3
    assert p.decode == [(1, 9)] and s.stats()["swap_preemptions"] == 1
    assert s.complete(p) == [1]                       # 1 had max_new 2: done, all free
    p = s.step()
    # 1 released 2, 1, 0 (last entry first) onto [3]: 0 is on top, then 1
    assert p.swap_in == [(0, 0), (1, 1)] and s.running == [2]
    assert p.decode == []                             # no work in the resuming step
    s.complete(p)
    p = s.step()
    assert p.decode == [(2, 9)]


def test_prefix_cached_prompts_start_past_their_cached_blocks():
    s = sched(nb=16, bs=4, tokens=64, chunk=64)
    s.add(1, 10, 1, tokens=list(range(10)))
    p = s.step()
    s.complete(p)                                     # finished, blocks 0, 1 stay cached
    s.add(2, 11, 1, tokens=list(range(8)) + [7, 7, 7])
    p = s.step()
    assert p.prefill == [(2, 8, 3)]                   # 8 positions reused
    assert s.a.tables[2][:2] == [0, 1]


def test_random_streams_conserve_blocks_and_finish_everything():
    rng = np.random.default_rng(4)
    for host in (0, 32):
        s = sched(nb=24, bs=4, seqs=6, tokens=24, chunk=8, host=host)
        for r in range(40):
            s.add(r, int(rng.integers(1, 30)), int(rng.integers(1, 12)))
        for _ in range(2000):
            p = s.step()
            s.complete(p)
            held = sum(len(t) for r, t in s.a.tables.items() if r not in s.a.swapped)
            assert s.a.stats()["num_used"] == held
            assert len(s.running) <= 6
            if s.stats()["finished"] == 40:
                break
        assert s.stats()["finished"] == 40
        assert s.a.stats()["num_free"] == 24

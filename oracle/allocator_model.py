"""Reference model of the host block allocator (plain Python, for tests only).

TEST INFRASTRUCTURE ONLY.  The product allocator is C++ behind the C-ABI; this
model states the same bookkeeping as directly as possible so that randomised
operation sequences can be replayed on both and compared.

Sources (page title, section):
  [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.1 — fixed-size blocks anywhere in
       the pool; allocate a block when a new token needs one; free a finished
       sequence's blocks at once; sequences may point at the same block.
  [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》 code example 1 — a
       sequence of n tokens needs ceil(n / block_size) blocks; asking for more
       than the pool holds is an error.
  [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §2.1 — a
       pre-allocated pool, per-block state (free / allocated / shareable),
       per-request block tables, copy-on-write for shared prefixes, and a
       free list popped from its end.

Semantics (identical in the C++ allocator):
  * The free list is a stack.  With ``free_order`` given, ``free_order[0]`` is
    handed out first, then ``free_order[1]``, ...  Without it, block 0 first.
  * ``append(seq, n)``: token at position ``pos`` lives in logical block
    ``pos // BS`` at offset ``pos % BS``; a new block is taken when
    ``pos % BS == 0``.  If the sequence's last block is partly filled and
    shared (refcount > 1), it is first replaced by a fresh block and the pair
    (old, new) is reported for a copy (copy-on-write); the old block loses one
    reference.  Slot = physical block * BS + offset.  All or nothing: if the
    pool cannot supply every block the call needs, nothing changes.
  * ``fork(parent, child)``: the child gets the parent's table and length; every
    block gains one reference.
  * ``free(seq)``: every block of the sequence loses one reference; blocks that
    reach zero are pushed back, last table entry first, so the sequence's first
    block is the next one handed out.
"""
from __future__ import annotations


class OutOfBlocks(Exception):
    pass


class AllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.stack = list(reversed(order))  # top of stack = end of list
        self.refcount = [0] * num_blocks
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}
        self.cow_copies = 0

    # -- helpers -----------------------------------------------------------
    def _take(self) -> int:
        b = self.stack.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    @staticmethod
    def blocks_for(num_tokens: int, block_size: int) -> int:
        return -(-num_tokens // block_size)

    # -- operations ---------------------------------------------------------
    def create(self, seq: int) -> None:
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lengths[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables:
            raise LookupError(parent)
        if child in self.tables:
            raise KeyError(child)
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def needed_blocks(self, seq: int, n: int) -> tuple[int, bool]:
        table, length = self.tables[seq], self.lengths[seq]
        bs = self.block_size
        fresh = self.blocks_for(length + n, bs) - self.blocks_for(length, bs)
        cow = n > 0 and length % bs != 0 and self.refcount[table[-1]] > 1
        return fresh + (1 if cow else 0), cow

    def append(self, seq: int, n: int):
        if seq not in self.tables:
            raise LookupError(seq)
        if n < 0:
            raise ValueError(n)
        need, cow = self.needed_blocks(seq, n)
        if need > len(self.stack):
            raise OutOfBlocks(f"need {need} blocks, {len(self.stack)} free")
        table = self.tables[seq]
        bs = self.block_size
        pairs = []
        if cow:
            src = table[-1]
            dst = self._take()
            self.refcount[src] -= 1
            table[-1] = dst
            pairs.append((src, dst))
            self.cow_copies += 1
        slots = []
        length = self.lengths[seq]
        for i in range(n):
            pos = length + i
            if pos % bs == 0:
                table.append(self._take())
            slots.append(table[pos // bs] * bs + pos % bs)
        self.lengths[seq] = length + n
        return slots, pairs

    def free(self, seq: int) -> None:
        if seq not in self.tables:
            raise LookupError(seq)
        for b in reversed(self.tables[seq]):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.stack.append(b)
        del self.tables[seq]
        del self.lengths[seq]

    # -- queries -------------------------------------------------------------
    def stats(self) -> dict:
        return {
            "num_blocks": self.num_blocks,
            "num_free": len(self.stack),
            "num_used": self.num_blocks - len(self.stack),
            "num_shared": sum(1 for r in self.refcount if r > 1),
            "cow_copies": self.cow_copies,
        }

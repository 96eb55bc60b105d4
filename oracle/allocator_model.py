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

Prefix cache (the pages: [VI] §2.1 allocation first reuses blocks that can be
shared with the request's prefix before taking free ones, keeps per-block
state free / allocated / shareable, and moves cold blocks out under an LRU
policy; [VI] §3 a switch that turns prompt sharing on; [NV] practical advice,
the prefix-cache hit rate as a serving metric).  The pages fix no key or
eviction rule; the reading taken here:
  * A block is registered once all its positions were appended with token
    ids (``append_tokens``) along an unbroken chain from position 0.  Its key
    is ``(parent, tokens of the block)``, where ``parent`` is the physical
    block of the previous logical block (-1 for the first).  Since the
    parent's own key names everything before it, a key names the whole prefix
    exactly.  A key that is already registered is not registered again; the
    sequence's chain stops there.  ``append`` (no token ids) stops the chain.
  * ``create_prefix(seq, tokens, max_cached)``: looks up the full blocks of
    ``tokens`` in order, at most ``max_cached // BS`` of them, and stops at the
    first miss.  Every hit joins the new sequence's table with one more
    reference; the length becomes ``hits * BS``.  Counters: every full block
    of ``tokens`` is queried, hits are counted.
  * Released blocks whose key is registered are not pushed on the free stack
    but appended to an LRU queue (they keep their contents for later hits);
    a hit on a queued block takes it out of the queue.
  * Taking a block pops the free stack; when it is empty, the oldest queued
    block is taken.  If that block is registered it is evicted: its key and
    the keys of all its registered descendants are dropped (their holders all
    hold it, so they are queued too; they stay in the queue, unregistered).
    Free blocks = stack + queue.

Swap (the pages: [NV] best practice 5, preemption moves a low-priority
request's KV cache out to CPU memory and back in when room returns; [VI] §2.1,
cold blocks migrate to CPU memory; [VI] §5, a CPU swap space).  Reading taken:
  * ``set_swap_space(n)`` gives a host pool of n blocks with its own free
    stack (host block 0 handed out first).
  * ``swap_out(seq)``: every table entry j in order gets a host block; the
    pairs (device block, host block) are returned for the copy; then the
    device blocks lose one reference each, last entry first, exactly as in
    ``free``.  The table now holds host blocks and the sequence is swapped.
    Sharing is not kept: a shared device block stays with its other holders
    and the swapped sequence owns a private host copy.
  * ``swap_in(seq)``: every entry j in order gets a device block (``_take``);
    pairs (host block, device block) are returned; the host blocks go back on
    the host stack, last entry first.  The new blocks are private and
    unregistered, so the sequence's prefix chain ends.
  * All or nothing: not enough host (or device) blocks raises OutOfBlocks
    with no change.  A swapped sequence cannot be appended to, forked or put
    in a batch table; freeing it returns its host blocks.

Host tier of the prefix cache (the pages: [VI] §2.1, cold blocks migrate to
CPU memory under an LRU policy).  Reading taken:
  * Entries are named by nodes: device block b is node b, host block h is
    node num_blocks + h; a key's parent is a node.
  * ``offload(max_blocks)`` walks the LRU queue from its oldest entry and
    moves each registered block, while host blocks are free and fewer than
    max_blocks moved, to a host block taken from the host stack: the entry
    keeps its key, its place among its parent's children and its children
    (whose keys now name the host node as parent).  The device block goes on
    the free stack.  Pairs (device block, host block) are returned for the
    copy.  Unregistered queued blocks are passed over.
  * ``create_prefix_ex(seq, tokens, max_cached)``: the chain of hits as in
    ``create_prefix``, where host entries may follow device ones.  The device
    hits are reused first (held); then each host hit, while a device block is
    free (counting the free stack and the queue after those holds) takes a
    block with ``_take`` and the entry moves back into it, its host block
    pushed on the host stack; pairs (host block, device block) are returned.
    ``create_prefix`` stops its chain at a host entry.
  * Dropping a subtree (eviction by ``_take``) drops its host entries too;
    their host blocks go back on the host stack lowest id on top.
  * ``set_swap_space`` is refused while entries are on the host.
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
        # prefix cache
        self.keys: dict[tuple, int] = {}          # (parent, tokens) -> block
        self.key_of: dict[int, tuple] = {}        # block -> its key
        self.children: dict[int, list[int]] = {}  # block -> registered children
        self.lru: list[int] = []                  # released cached blocks, oldest first
        self.chain: dict[int, bool] = {}          # seq -> every position has token ids
        self.pending: dict[int, list[int]] = {}   # seq -> tokens of its partial block
        self.parent: dict[int, int] = {}          # seq -> block of its last full block
        self.queried_blocks = 0
        self.hit_blocks = 0
        # swap space
        self.host_stack: list[int] = []
        self.num_host_blocks = 0
        self.swapped: set[int] = set()
        self.swap_out_blocks = 0
        self.swap_in_blocks = 0
        # host tier of the prefix cache
        self.offloaded_blocks = 0
        self.reloaded_blocks = 0

    # -- helpers -----------------------------------------------------------
    def _take(self) -> int:
        if self.stack:
            b = self.stack.pop()
        else:
            b = self.lru.pop(0)
            if b in self.key_of:
                dropped = []
                self._unregister(b, dropped=dropped)
                for node in sorted(dropped, reverse=True):  # lowest id on top
                    self.host_stack.append(node - self.num_blocks)
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def _unregister(self, b: int, parent_going: bool = False, dropped=None) -> None:
        for c in self.children.pop(b, []):
            self._unregister(c, parent_going=True, dropped=dropped)
        key = self.key_of.pop(b)
        del self.keys[key]
        if key[0] >= 0 and not parent_going:
            self.children[key[0]].remove(b)
        if b >= self.num_blocks:
            dropped.append(b)

    def _move(self, src: int, dst: int) -> None:
        """Entry ``src`` becomes node ``dst``; its children's keys follow."""
        key = self.key_of.pop(src)
        self.keys[key] = dst
        self.key_of[dst] = key
        if key[0] >= 0:
            sib = self.children[key[0]]
            sib[sib.index(src)] = dst
        kids = self.children.pop(src, [])
        for c in kids:
            old = self.key_of[c]
            del self.keys[old]
            new = (dst, old[1])
            self.keys[new] = c
            self.key_of[c] = new
        if kids:
            self.children[dst] = kids

    def num_host_cached(self) -> int:
        return sum(1 for n in self.key_of if n >= self.num_blocks)

    def _num_free(self) -> int:
        return len(self.stack) + len(self.lru)

    @staticmethod
    def blocks_for(num_tokens: int, block_size: int) -> int:
        return -(-num_tokens // block_size)

    # -- operations ---------------------------------------------------------
    def create(self, seq: int) -> None:
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lengths[seq] = 0
        self.chain[seq] = True
        self.pending[seq] = []
        self.parent[seq] = -1

    def create_prefix(self, seq: int, tokens, max_cached: int) -> int:
        """New sequence starting with the cached blocks of ``tokens``;
        returns the number of cached positions."""
        return self._create_prefix(seq, tokens, max_cached, host=False)[0]

    def create_prefix_ex(self, seq: int, tokens, max_cached: int, cap: int | None = None):
        """create_prefix that brings host-tier hits back; returns (cached
        positions, pairs (host block, device block))."""
        return self._create_prefix(seq, tokens, max_cached, host=True, cap=cap)

    def _create_prefix(self, seq, tokens, max_cached, host, cap=None):
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        self.queried_blocks += len(tokens) // bs
        chain, parent = [], -1
        for j in range(min(len(tokens), max(max_cached, 0)) // bs):
            b = self.keys.get((parent, tuple(tokens[j * bs:(j + 1) * bs])))
            if b is None or (b >= self.num_blocks and not host):
                break
            chain.append(b)
            parent = b
        dev = [b for b in chain if b < self.num_blocks]
        assert chain[:len(dev)] == dev  # host entries only after device ones
        avail = self._num_free() - sum(1 for b in dev if self.refcount[b] == 0)
        n_host = min(len(chain) - len(dev), max(avail, 0),
                     len(chain) if cap is None else cap) if host else 0
        for b in dev:
            if self.refcount[b] == 0:
                self.lru.remove(b)
            self.refcount[b] += 1
        table, pairs = list(dev), []
        for node in chain[len(dev):len(dev) + n_host]:
            d = self._take()
            self._move(node, d)
            self.host_stack.append(node - self.num_blocks)
            pairs.append((node - self.num_blocks, d))
            table.append(d)
        self.reloaded_blocks += n_host
        self.hit_blocks += len(table)
        self.tables[seq] = table
        self.lengths[seq] = len(table) * bs
        self.chain[seq] = True
        self.pending[seq] = []
        self.parent[seq] = table[-1] if table else -1
        return len(table) * bs, pairs

    def offload(self, max_blocks: int):
        """Move up to max_blocks of the oldest queued registered blocks to
        the host tier; returns pairs (device block, host block)."""
        pairs = []
        for b in list(self.lru):
            if len(pairs) >= max_blocks or not self.host_stack:
                break
            if b not in self.key_of:
                continue
            h = self.host_stack.pop()
            self._move(b, self.num_blocks + h)
            self.lru.remove(b)
            self.stack.append(b)
            pairs.append((b, h))
        self.offloaded_blocks += len(pairs)
        return pairs

    def host_stats(self) -> dict:
        return {"host_cached_blocks": self.num_host_cached(),
                "offloaded_blocks": self.offloaded_blocks,
                "reloaded_blocks": self.reloaded_blocks}

    def set_swap_space(self, num_host_blocks: int) -> None:
        if self.swapped:
            raise ValueError("sequences are swapped out")
        if self.num_host_cached():
            raise ValueError("prefix-cache entries are on the host")
        self.num_host_blocks = int(num_host_blocks)
        self.host_stack = list(range(self.num_host_blocks - 1, -1, -1))

    def swap_out(self, seq: int):
        if seq not in self.tables:
            raise LookupError(seq)
        if seq in self.swapped:
            raise ValueError("already swapped out")
        table = self.tables[seq]
        if len(table) > len(self.host_stack):
            raise OutOfBlocks(f"need {len(table)} host blocks, {len(self.host_stack)} free")
        host = [self.host_stack.pop() for _ in table]
        pairs = list(zip(table, host))
        for b in reversed(table):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                if b in self.key_of:
                    self.lru.append(b)
                else:
                    self.stack.append(b)
        self.tables[seq] = host
        self.swapped.add(seq)
        self.swap_out_blocks += len(host)
        return pairs

    def swap_in(self, seq: int):
        if seq not in self.tables:
            raise LookupError(seq)
        if seq not in self.swapped:
            raise ValueError("not swapped out")
        host = self.tables[seq]
        if len(host) > self._num_free():
            raise OutOfBlocks(f"need {len(host)} blocks, {self._num_free()} free")
        dev = [self._take() for _ in host]
        pairs = list(zip(host, dev))
        for h in reversed(host):
            self.host_stack.append(h)
        self.tables[seq] = dev
        self.swapped.discard(seq)
        self.chain[seq] = False
        self.pending[seq] = []
        self.swap_in_blocks += len(dev)
        return pairs

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables:
            raise LookupError(parent)
        if parent in self.swapped:
            raise ValueError("swapped out")
        if child in self.tables:
            raise KeyError(child)
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        self.chain[child] = self.chain[parent]
        self.pending[child] = list(self.pending[parent])
        self.parent[child] = self.parent[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def needed_blocks(self, seq: int, n: int) -> tuple[int, bool]:
        table, length = self.tables[seq], self.lengths[seq]
        bs = self.block_size
        fresh = self.blocks_for(length + n, bs) - self.blocks_for(length, bs)
        cow = n > 0 and length % bs != 0 and self.refcount[table[-1]] > 1
        return fresh + (1 if cow else 0), cow

    def append(self, seq: int, n: int, tokens=None):
        """Append n positions (with their token ids when ``tokens`` is given:
        see the prefix cache above)."""
        if seq not in self.tables:
            raise LookupError(seq)
        if n < 0:
            raise ValueError(n)
        if tokens is not None and len(tokens) != n:
            raise ValueError("len(tokens) != n")
        if seq in self.swapped:
            raise ValueError("swapped out")
        need, cow = self.needed_blocks(seq, n)
        if need > self._num_free():
            raise OutOfBlocks(f"need {need} blocks, {self._num_free()} free")
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
        if tokens is None and n > 0:
            self.chain[seq] = False
            self.pending[seq] = []
        for i in range(n):
            pos = length + i
            if pos % bs == 0:
                table.append(self._take())
            slots.append(table[pos // bs] * bs + pos % bs)
            if tokens is not None and self.chain[seq]:
                self.pending[seq].append(int(tokens[i]))
                if pos % bs == bs - 1:
                    self._register(seq, table[pos // bs])
        self.lengths[seq] = length + n
        return slots, pairs

    def _register(self, seq: int, b: int) -> None:
        key = (self.parent[seq], tuple(self.pending[seq]))
        self.pending[seq] = []
        if key in self.keys:
            self.chain[seq] = False
            return
        self.keys[key] = b
        self.key_of[b] = key
        if key[0] >= 0:
            self.children.setdefault(key[0], []).append(b)
        self.parent[seq] = b

    def free(self, seq: int) -> None:
        if seq not in self.tables:
            raise LookupError(seq)
        if seq in self.swapped:
            for h in reversed(self.tables[seq]):
                self.host_stack.append(h)
            self.swapped.discard(seq)
            self.tables[seq] = []
        for b in reversed(self.tables[seq]):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                if b in self.key_of:
                    self.lru.append(b)
                else:
                    self.stack.append(b)
        for d in (self.tables, self.lengths, self.chain, self.pending, self.parent):
            del d[seq]

    # -- queries -------------------------------------------------------------
    def stats(self) -> dict:
        return {
            "num_blocks": self.num_blocks,
            "num_free": self._num_free(),
            "num_used": self.num_blocks - self._num_free(),
            "num_shared": sum(1 for r in self.refcount if r > 1),
            "cow_copies": self.cow_copies,
        }

    def prefix_stats(self) -> dict:
        return {
            "queried_blocks": self.queried_blocks,
            "hit_blocks": self.hit_blocks,
            "cached_blocks": len(self.keys),
            "cached_free_blocks": sum(1 for b in self.lru if b in self.key_of),
        }

    def swap_stats(self) -> dict:
        return {
            "num_host_blocks": self.num_host_blocks,
            "num_host_free": len(self.host_stack),
            "swapped_seqs": len(self.swapped),
            "swap_out_blocks": self.swap_out_blocks,
            "swap_in_blocks": self.swap_in_blocks,
        }

"""Reference model of the continuous-batching scheduler (plain Python, tests only).

TEST INFRASTRUCTURE ONLY.  The product scheduler is C++ behind the C-ABI; this
model states the same policy as directly as possible so that randomised
request streams can be replayed on both and every step's plan compared.

Sources (page title, section):
  [VE] 《加速 LLM 推理：深入了解 vLLM 引擎》 §3.2 — continuous batching: requests
       join the running batch at every iteration and leave as soon as they
       finish, instead of waiting for the whole batch.
  [VI] 《vLLM大模型推理引擎：高效解决显存碎片与请求排队难题》 §1 — one iteration
       mixes prefill and decode; §2.2 — new requests enter a pending queue and
       get their first blocks when admitted; each cycle collects runnable
       requests, merges new ones, runs, updates block state; finished requests
       release their resources at once.
  [NV] 《Nano-vLLM 原理：vLLM 风格推理引擎的实现机制》 best practice 5 — first-come
       first-served admission, and preemption that moves a request's KV cache to
       CPU memory when a request cannot get resources, bringing it back later.

Policy (the pages leave the details open; this is the reading, identical in
the C++ scheduler):
  * A request has a prompt of n positions and asks for max_new generated
    tokens.  Its prompt is written in chunks (chunked prefill); the step that
    writes the last chunk yields the first generated token; every later step
    appends that token's position and decodes the next one.  When max_new
    tokens exist it finishes and its blocks are freed.
  * Each step, in this order:
    1. Decode set: running requests whose prompt is complete, in admission
       order; each needs one position.  While the pool cannot hold those
       positions, the most recently admitted running request is preempted:
       swapped out if the host pool has room for its blocks, otherwise
       dropped back to the front of the waiting queue to start over
       (recompute).
    2. The decode positions are appended.
    3. The step's token budget (max_batched_tokens minus the decode count)
       goes to running requests still in their prompt, in admission order,
       each getting min(rest of prompt, budget, max_prefill_chunk) positions
       while the pool can hold them.
    4. Swapped requests come back in arrival order while fewer than
       max_num_seqs run and the pool holds their blocks; they do no work in
       the step that resumes them.
    5. Waiting requests are admitted in queue order while fewer than
       max_num_seqs run, budget remains and the pool holds their first chunk.
       A request with token ids first reuses its cached prompt blocks
       (leaving at least its last position to compute).
  * Parallel sampling ([VE] §3.1: the outputs drawn from one prompt share its
    KV blocks, copy-on-write where they diverge).  A request may ask for n
    samples.  It runs as one sequence until its prompt is written; completing
    that step forks samples 2..n from it, so all n hold the prompt's blocks.
    Afterwards its n sequences decode in the same steps, adjacent in the
    decode list (the request's own id first), and are preempted (all swapped,
    or all dropped and the request restarted), resumed and finished together.
    max_num_seqs counts sequences; a request holds n of them from admission.
  * A request is refused when, alone in the pool, it might not finish:
    n * ceil((n_prompt + max_new - 1) / block_size) blocks (+1 with samples:
    the decode-set check counts a fork's shared partial block once more than
    the copies it takes) must fit the pool, or it would be preempted and
    restarted for ever.  Samples hold private copies after a swap, hence the
    factor n.
"""
from __future__ import annotations

import dataclasses
from collections import deque

from oracle.allocator_model import AllocatorModel, OutOfBlocks


@dataclasses.dataclass
class Request:
    rid: int
    n_prompt: int
    max_new: int
    tokens: list | None
    order: int              # arrival order
    done: int = 0           # prompt positions written
    generated: int = 0
    state: str = "waiting"  # waiting | running | swapped | finished
    samples: list = dataclasses.field(default_factory=list)  # ids of samples 2..n
    forked: bool = False    # the samples exist in the allocator

    def seqs(self) -> list:
        """The sequence ids that hold blocks now."""
        return [self.rid] + (self.samples if self.forked else [])


@dataclasses.dataclass
class Plan:
    decode: list            # [(sequence id, context length after the append)]
    prefill: list           # [(rid, start position, chunk length)]
    swap_out: list          # [(device block, host block)], all swapped-out requests
    swap_in: list           # [(host block, device block)]
    cow: list               # [(src, dst)]
    slots: list             # decode slots (one per decode entry) then prefill slots in order
    preempted: list         # request ids dropped back to waiting (recompute)


class SchedulerModel:
    def __init__(self, alloc: AllocatorModel, max_num_seqs: int, max_batched_tokens: int,
                 max_prefill_chunk: int):
        if min(max_num_seqs, max_batched_tokens, max_prefill_chunk) < 1 or \
                max_batched_tokens < max_num_seqs:
            raise ValueError("bad scheduler sizes")
        self.a = alloc
        self.max_num_seqs = max_num_seqs
        self.max_batched_tokens = max_batched_tokens
        self.max_prefill_chunk = max_prefill_chunk
        self.reqs: dict[int, Request] = {}
        self.sample_of: dict[int, int] = {}
        self.waiting: deque[int] = deque()
        self.running: list[int] = []
        self.swapped: list[int] = []
        self.arrivals = 0
        self.swap_preemptions = 0
        self.recompute_preemptions = 0
        self.finished = 0
        self.forked_samples = 0

    def _taken(self, x: int) -> bool:
        return x in self.reqs or x in self.sample_of

    def add(self, rid: int, n_prompt: int, max_new: int, tokens=None, samples=()) -> None:
        samples = [int(x) for x in samples]
        if n_prompt < 1 or max_new < 1 or 1 + len(samples) > self.max_num_seqs:
            raise ValueError("bad request")
        ids = [rid] + samples
        if len(set(ids)) != len(ids) or any(self._taken(x) for x in ids):
            raise ValueError("id taken")
        if tokens is not None and len(tokens) != n_prompt:
            raise ValueError("len(tokens) != n_prompt")
        # alone in the pool it must be able to finish (see the policy above)
        per_seq = -(-(n_prompt + max_new - 1) // self.a.block_size)
        if per_seq * (1 + len(samples)) + (1 if samples else 0) > self.a.num_blocks:
            raise ValueError("the request cannot fit the pool")
        self.reqs[rid] = Request(rid, n_prompt, max_new,
                                 None if tokens is None else [int(t) for t in tokens],
                                 self.arrivals, samples=samples)
        for x in samples:
            self.sample_of[x] = rid
        self.arrivals += 1
        self.waiting.append(rid)

    def _running_seqs(self) -> int:
        return sum(1 + len(self.reqs[r].samples) for r in self.running)

    # -- one step ---------------------------------------------------------------
    def _free_blocks(self) -> int:
        return self.a._num_free()

    def _decode_need(self, ids) -> int:
        return sum(self.a.needed_blocks(x, 1)[0] for r in ids for x in self.reqs[r].seqs())

    def _blocks(self, r: Request) -> int:
        return sum(len(self.a.tables[x]) for x in r.seqs())

    def _preempt(self, rid: int, plan: Plan) -> None:
        """Preempt request rid with all its sequences: each swapped out (a
        private host copy per sequence) when the host pool holds them all,
        else all freed and the request restarted from its prompt."""
        r = self.reqs[rid]
        self.running.remove(rid)
        if self._blocks(r) <= len(self.a.host_stack):
            for x in r.seqs():
                plan.swap_out += self.a.swap_out(x)
            r.state = "swapped"
            self.swapped.append(rid)
            self.swapped.sort(key=lambda x: self.reqs[x].order)
            self.swap_preemptions += 1
        else:
            for x in r.seqs():
                self.a.free(x)
            r.state, r.done, r.generated, r.forked = "waiting", 0, 0, False
            self.waiting.appendleft(rid)
            plan.preempted.append(rid)
            self.recompute_preemptions += 1

    def step(self) -> Plan:
        a, bs = self.a, self.a.block_size
        plan = Plan([], [], [], [], [], [], [])
        # 1. decode set, preempting the newest running request while it does not fit
        while True:
            dec = [r for r in self.running if self.reqs[r].done == self.reqs[r].n_prompt]
            if self._decode_need(dec) <= self._free_blocks() or not self.running:
                break
            self._preempt(self.running[-1], plan)
        # 2. decode positions, each request's sequences in a row
        for rid in dec:
            for x in self.reqs[rid].seqs():
                s, p = a.append(x, 1)
                plan.slots += s
                plan.cow += p
                plan.decode.append((x, a.lengths[x]))
        budget = self.max_batched_tokens - len(plan.decode)
        # 3. prompts in progress
        for rid in list(self.running):
            r = self.reqs[rid]
            if r.done == r.n_prompt:
                continue
            c = min(r.n_prompt - r.done, budget, self.max_prefill_chunk)
            if c <= 0 or a.needed_blocks(rid, c)[0] > self._free_blocks():
                break
            self._append_prompt(r, c, plan)
            budget -= c
        # 4. swapped requests come back
        while self.swapped:
            r = self.reqs[self.swapped[0]]
            if self._running_seqs() + 1 + len(r.samples) > self.max_num_seqs or \
                    self._blocks(r) > self._free_blocks():
                break
            for x in r.seqs():
                plan.swap_in += a.swap_in(x)
            self.swapped.pop(0)
            r.state = "running"
            self.running.append(r.rid)
        # 5. admissions
        while self.waiting and budget > 0:
            r = self.reqs[self.waiting[0]]
            if self._running_seqs() + 1 + len(r.samples) > self.max_num_seqs:
                break
            if r.tokens is not None:
                cached = a.create_prefix(r.rid, r.tokens, r.n_prompt - 1)
            else:
                a.create(r.rid)
                cached = 0
            c = min(r.n_prompt - cached, budget, self.max_prefill_chunk)
            if a.needed_blocks(r.rid, c)[0] > self._free_blocks():
                a.free(r.rid)  # not admitted: its cached blocks go back
                break
            self.waiting.popleft()
            r.done, r.state = cached, "running"
            self.running.append(r.rid)
            self._append_prompt(r, c, plan)
            budget -= c
        return plan

    def _append_prompt(self, r: Request, c: int, plan: Plan) -> None:
        toks = None if r.tokens is None else r.tokens[r.done:r.done + c]
        s, p = self.a.append(r.rid, c, tokens=toks)
        plan.slots += s
        plan.cow += p
        plan.prefill.append((r.rid, r.done, c))
        r.done += c

    def complete(self, plan: Plan) -> list:
        """The step ran: fork the samples of requests whose prompt it wrote,
        count its tokens (one per request per step: its samples advance
        together), retire finished requests (freed at once).  Returns the
        finished sequence ids: per request in running order, its own id, then
        its samples'."""
        for rid, start, c in plan.prefill:
            r = self.reqs[rid]
            if start + c == r.n_prompt and r.state == "running" and r.samples:
                for x in r.samples:
                    self.a.fork(rid, x)
                r.forked = True
                self.forked_samples += len(r.samples)
        for rid in dict.fromkeys(self.sample_of.get(x, x) for x, _ in plan.decode):
            self.reqs[rid].generated += 1
        for rid, start, c in plan.prefill:
            r = self.reqs[rid]
            if start + c == r.n_prompt and r.state == "running":
                r.generated += 1
        fin = []
        for rid in list(self.running):
            r = self.reqs[rid]
            if r.generated >= r.max_new:
                for x in r.seqs():
                    self.a.free(x)
                    fin.append(x)
                self.running.remove(rid)
                r.state = "finished"
                self.finished += 1
        return fin

    def stats(self) -> dict:
        return {"waiting": len(self.waiting), "running": len(self.running),
                "swapped": len(self.swapped), "running_seqs": self._running_seqs(),
                "finished": self.finished,
                "swap_preemptions": self.swap_preemptions,
                "recompute_preemptions": self.recompute_preemptions,
                "forked_samples": self.forked_samples}

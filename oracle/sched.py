"""CPU oracle for the slot scheduler that drives the paged-attention kernels step by step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the native library and imports nothing from it.

Sources (cited by title and section):
  [实战]  "Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎", §连续批处理：吞吐与延迟的平衡:
          the batch is a fixed number of slots, one request per slot; a slot moves through
          waiting -> prefill -> decode -> done; a finished slot takes the next queued
          request into prefill; prefill runs on its own while decode runs every active
          slot together; prefill and decode are kept apart so that a long prefill does not
          hold up the decode of short requests.
  [guide] "tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §PagedAttention: pages are
          taken only when needed; §推理流程：从Prefill到Decode: a sequence's new K/V joins
          the cache before it attends, one token per decode step.
  [实战]  §内存池管理: a preallocated pool hands pages out and takes them back when a
          request ends.

What a step does (this oracle's reading):
  1. Retire: a request that has produced its max_new tokens, or that the caller finished,
     returns its pages to the pool and frees its slot.
  2. Admit: while a slot is free, the oldest waiting request enters it (lowest free slot
     first), provided the pool's free pages, less the pages already promised to admitted
     requests, cover its worst case, ceil((prompt + max_new - 1) / block_size) pages.
     The queue is served strictly in order: a request that does not fit stops admission.
  3. Kind: a prefill step if some slot is prefilling and either no slot is decoding or
     the previous step was not a prefill step; else a decode step if some slot is
     decoding; else idle.  So prefill and decode steps alternate while both are pending.
  4. Prefill step: prefilling slots in admission order take prompt tokens, each as many
     as it has left, until the step's budget of prefill_chunk tokens is spent.  A slot
     whose prompt is complete has produced its first token: it decodes from the next step
     (or is done, if max_new is 1).
  5. Decode step: every decoding slot appends its last token (context + 1) and produces
     the next.
  Pages are taken from the pool only for the tokens a step appends (block b of a request
  is allocated in the step that first writes a token into it).

Invariants and closed cases pinned in tests/test_oracle_sched.py.
"""

from __future__ import annotations

from dataclasses import dataclass, field

IDLE, PREFILL, DECODE = 0, 1, 2


@dataclass
class Request:
    rid: int
    prompt: int
    max_new: int
    order: int                      # admission order (set when admitted)
    slot: int = -1
    cached: int = 0                 # tokens whose K/V are in the cache
    generated: int = 0              # tokens produced so far
    pages: list = field(default_factory=list)
    stop: bool = False              # finished by the caller

    def reserve(self, bs: int) -> int:
        return -(-(self.prompt + self.max_new - 1) // bs)

    def done(self) -> bool:
        return self.stop or self.generated >= self.max_new


@dataclass
class Plan:
    kind: int
    rows: list          # per row: (rid, slot, ctx_after, n_new, block-table row as a list)
    finished: list      # request ids retired at the start of this step


class Pool:
    """Free-page stack with the same hand-out order as any LIFO list: the oracle's own."""

    def __init__(self, num_pages: int):
        self.free = list(range(num_pages - 1, -1, -1))

    def take(self) -> int:
        return self.free.pop()

    def give(self, pages) -> None:
        for p in pages:
            self.free.append(p)


class Scheduler:
    def __init__(self, num_slots: int, block_size: int, max_blocks: int, prefill_chunk: int,
                 pool: Pool):
        self.num_slots, self.bs = num_slots, block_size
        self.max_blocks, self.chunk = max_blocks, prefill_chunk
        self.pool = pool
        self.queue: list[Request] = []
        self.active: list[Request] = []   # admission order
        self.last = IDLE
        self.admitted = 0

    def submit(self, rid: int, prompt: int, max_new: int) -> bool:
        if prompt < 1 or max_new < 1:
            return False
        r = Request(rid, prompt, max_new, order=-1)
        if r.reserve(self.bs) > self.max_blocks:
            return False
        if any(x.rid == rid for x in self.queue + self.active):
            return False
        self.queue.append(r)
        return True

    def finish(self, rid: int) -> bool:
        for i, r in enumerate(self.queue):
            if r.rid == rid:
                del self.queue[i]
                return True
        for r in self.active:
            if r.rid == rid:
                r.stop = True
                return True
        return False

    def _promised(self) -> int:
        return sum(r.reserve(self.bs) - len(r.pages) for r in self.active)

    def _grow(self, r: Request, tokens: int) -> None:
        need = -(-tokens // self.bs)
        while len(r.pages) < need:
            r.pages.append(self.pool.take())

    def step(self) -> Plan:
        # 1. retire
        finished = []
        keep = []
        for r in self.active:
            if r.done():
                self.pool.give(r.pages)
                finished.append(r.rid)
            else:
                keep.append(r)
        self.active = keep
        # 2. admit, oldest first, lowest free slot first
        while self.queue and len(self.active) < self.num_slots:
            r = self.queue[0]
            if r.reserve(self.bs) > len(self.pool.free) - self._promised():
                break
            self.queue.pop(0)
            used = {x.slot for x in self.active}
            r.slot = min(s for s in range(self.num_slots) if s not in used)
            r.order = self.admitted
            self.admitted += 1
            self.active.append(r)
        # 3. kind
        pre = [r for r in self.active if r.cached < r.prompt]
        dec = [r for r in self.active if r.cached >= r.prompt]
        if pre and (not dec or self.last != PREFILL):
            kind = PREFILL
        elif dec:
            kind = DECODE
        else:
            kind = IDLE
        # 4./5. rows
        rows = []
        if kind == PREFILL:
            budget = self.chunk
            for r in pre:
                n = min(r.prompt - r.cached, budget)
                if n == 0:
                    break
                budget -= n
                self._grow(r, r.cached + n)
                r.cached += n
                if r.cached == r.prompt:
                    r.generated = 1
                rows.append((r.rid, r.slot, r.cached, n, list(r.pages)))
        elif kind == DECODE:
            for r in dec:
                self._grow(r, r.cached + 1)
                r.cached += 1
                r.generated += 1
                rows.append((r.rid, r.slot, r.cached, 1, list(r.pages)))
        self.last = kind
        return Plan(kind, rows, finished)

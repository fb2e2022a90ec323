"""Pins for the slot-scheduler oracle (oracle/sched.py): hand-traced closed cases and
invariants checked over seeded random request streams.  CPU only."""

from __future__ import annotations

import numpy as np

from oracle import sched as S


def test_one_request_hand_traced():
    # prompt 40, 3 new tokens, pages of 16, prefill budget 32 tokens per step
    sc = S.Scheduler(num_slots=2, block_size=16, max_blocks=8, prefill_chunk=32,
                     pool=S.Pool(10))
    assert sc.submit(7, 40, 3)
    want = [
        (S.PREFILL, [(7, 0, 32, 32, [0, 1])], []),
        (S.PREFILL, [(7, 0, 40, 8, [0, 1, 2])], []),   # prompt done: first token produced
        (S.DECODE, [(7, 0, 41, 1, [0, 1, 2])], []),
        (S.DECODE, [(7, 0, 42, 1, [0, 1, 2])], []),    # third token produced
        (S.IDLE, [], [7]),
    ]
    for kind, rows, fin in want:
        p = sc.step()
        assert (p.kind, p.rows, p.finished) == (kind, rows, fin)
    assert sorted(sc.pool.free) == list(range(10))


def test_single_new_token_is_done_after_prefill():
    sc = S.Scheduler(1, 16, 4, 64, S.Pool(4))
    sc.submit(1, 16, 1)
    p = sc.step()
    assert p.kind == S.PREFILL and p.rows == [(1, 0, 16, 16, [0])]
    p = sc.step()
    assert (p.kind, p.rows, p.finished) == (S.IDLE, [], [1])


def test_slots_bound_concurrency_and_freed_slot_is_reused():
    sc = S.Scheduler(2, 16, 4, 1000, S.Pool(64))
    for rid in (10, 11, 12):
        sc.submit(rid, 5, 2)
    p = sc.step()                     # 10 and 11 admitted, prefilled together
    assert p.kind == S.PREFILL and [r[:4] for r in p.rows] == [(10, 0, 5, 5), (11, 1, 5, 5)]
    p = sc.step()                     # both decode; 12 still waits
    assert p.kind == S.DECODE and [r[0] for r in p.rows] == [10, 11] and sc.queue[0].rid == 12
    p = sc.step()                     # both retired, 12 takes slot 0
    assert p.finished == [10, 11] and p.kind == S.PREFILL and p.rows[0][:2] == (12, 0)


def test_prefill_and_decode_alternate():
    sc = S.Scheduler(4, 16, 64, 100, S.Pool(256))
    sc.submit(1, 10, 50)
    sc.step()                          # prefill of 1: it decodes from now on
    sc.submit(2, 450, 5)              # a long prompt arrives
    # the step after a prefill step decodes, then the kinds take turns
    kinds = [sc.step().kind for _ in range(10)]
    assert kinds == [S.DECODE, S.PREFILL] * 5
    # the long prompt advanced by the 100-token budget per prefill step
    assert sc.active[1].cached == 450 and sc.active[0].generated == 1 + 5


def test_budget_splits_across_prompts_in_admission_order():
    sc = S.Scheduler(3, 16, 64, 50, S.Pool(256))
    for rid, n in ((1, 30), (2, 30), (3, 30)):
        sc.submit(rid, n, 4)
    p = sc.step()
    assert [r[:4] for r in p.rows] == [(1, 0, 30, 30), (2, 1, 20, 20)]
    # nothing decodes yet (1 has finished its prompt, so the next step decodes it)
    p = sc.step()
    assert p.kind == S.DECODE and [r[:4] for r in p.rows] == [(1, 0, 31, 1)]
    p = sc.step()
    assert p.kind == S.PREFILL and [r[:4] for r in p.rows] == [(2, 1, 30, 10), (3, 2, 30, 30)]


def test_admission_waits_for_pages_in_queue_order():
    # pool of 6 pages, bs 16: a request of 60 + 20 needs ceil(79/16) = 5 pages
    sc = S.Scheduler(4, 16, 16, 1000, S.Pool(6))
    sc.submit(1, 60, 20)
    sc.submit(2, 10, 2)               # would fit (1 page) but may not overtake
    sc.submit(3, 60, 20)
    p = sc.step()
    assert [r[0] for r in p.rows] == [1, 2]   # 1 (5 pages promised) + 2 (1 page) = 6
    assert [r.rid for r in sc.queue] == [3]
    while 1 in [r.rid for r in sc.active]:
        sc.step()
    assert [r.rid for r in sc.active] == [3]
    # never more pages promised than the pool holds
    assert sc._promised() + sum(len(r.pages) for r in sc.active) <= 6


def test_finish_early_and_from_the_queue():
    sc = S.Scheduler(1, 16, 8, 64, S.Pool(8))
    sc.submit(1, 20, 100)
    sc.submit(2, 20, 3)
    sc.step(); sc.step()
    assert sc.finish(2) and [r.rid for r in sc.queue] == []
    assert sc.finish(1)
    p = sc.step()
    assert p.finished == [1] and p.kind == S.IDLE and len(sc.pool.free) == 8
    assert not sc.finish(1)


def test_rejects_what_can_never_run():
    sc = S.Scheduler(2, 16, 4, 64, S.Pool(100))
    assert not sc.submit(1, 60, 6)    # ceil(65/16) = 5 blocks > a 4-entry block table
    assert sc.submit(1, 60, 5)        # ceil(64/16) = 4 fits exactly
    assert not sc.submit(1, 3, 3)     # duplicate id
    assert not sc.submit(2, 0, 3) and not sc.submit(3, 5, 0)


def _stream(seed, n, slots, bs, max_blocks, chunk, pages):
    rng = np.random.default_rng(seed)
    sc = S.Scheduler(slots, bs, max_blocks, chunk, S.Pool(pages))
    reqs = {}
    for rid in range(n):
        p, m = int(rng.integers(1, 300)), int(rng.integers(1, 40))
        if sc.submit(rid, p, m):
            reqs[rid] = (p, m)
    return sc, reqs


def test_invariants_over_random_streams():
    for seed in range(12):
        bs = 16 if seed % 2 else 32
        total = 40 + 13 * seed
        sc, reqs = _stream(seed, 60, slots=1 + seed % 7, bs=bs, max_blocks=24,
                           chunk=37 + 50 * seed, pages=total)
        prefilled = {r: 0 for r in reqs}
        produced = {r: 0 for r in reqs}
        seen_pages = {}
        last = S.IDLE
        finished = []
        for _ in range(100000):
            # decoding requests that the step will keep (a done one is retired first)
            decoding = [r.rid for r in sc.active if r.cached >= r.prompt and not r.done()]
            p = sc.step()
            finished += p.finished
            if p.kind == S.PREFILL and last == S.PREFILL:
                assert not decoding          # two prefill steps in a row only if none decodes
            if p.kind == S.DECODE:
                assert [row[0] for row in p.rows] == decoding   # every decoding slot, in order
            held = [pg for r in sc.active for pg in r.pages]
            assert len(held) == len(set(held))                   # no page in two requests
            assert len(held) + len(sc.pool.free) == total        # every page accounted for
            assert sc._promised() <= len(sc.pool.free)           # promises can be kept
            slots = [row[1] for row in p.rows]
            assert len(slots) == len(set(slots)) and all(0 <= s < sc.num_slots for s in slots)
            if p.kind == S.PREFILL:
                assert sum(row[3] for row in p.rows) <= sc.chunk
            for rid, slot, ctx, n, table in p.rows:
                assert len(table) == -(-ctx // sc.bs) <= sc.max_blocks
                prev = seen_pages.get(rid, [])
                assert table[:len(prev)] == prev                 # a block table only grows
                seen_pages[rid] = table
                if p.kind == S.PREFILL:
                    prefilled[rid] += n
                    produced[rid] += ctx == reqs[rid][0]
                else:
                    assert n == 1 and ctx > reqs[rid][0]
                    produced[rid] += 1
            last = p.kind
            if p.kind == S.IDLE and not sc.queue and not sc.active:
                break
        assert sorted(finished) == sorted(reqs)
        for rid, (prompt, m) in reqs.items():
            assert prefilled[rid] == prompt and produced[rid] == m
        assert sorted(sc.pool.free) == list(range(total))

"""The native slot scheduler (pa_sched_*) against the oracle (oracle/sched.py), decision
by decision: every step's kind, rows (request, slot, context, new tokens, block table)
and retirements must be identical, over seeded request streams with arrivals and early
finishes between steps.  Host logic only: CPU, no device."""

from __future__ import annotations

import numpy as np
import pytest

import paged_kv_attention_31_amd as pa
from oracle import sched as S


def _same(native, oracle_plan, max_blocks):
    assert native.kind == oracle_plan.kind
    assert native.finished.tolist() == oracle_plan.finished
    rows = oracle_plan.rows
    assert native.req_ids.tolist() == [r[0] for r in rows]
    assert native.slots.tolist() == [r[1] for r in rows]
    assert native.ctx_lens.tolist() == [r[2] for r in rows]
    assert np.diff(native.cu_new_lens).tolist() == [r[3] for r in rows]
    assert native.cu_new_lens[0] == 0
    for k, r in enumerate(rows):
        table = r[4]
        assert native.block_tables[k, :len(table)].tolist() == table
        assert np.all(native.block_tables[k, len(table):] == -1)
    if rows:
        assert native.max_ctx_len == max(r[2] for r in rows)
        assert native.max_new_len == max(r[3] for r in rows)


def _drive(seed, slots, bs, max_blocks, chunk, pages, n_req, arrivals, finishes):
    rng = np.random.default_rng(seed)
    pool = pa.PagePool(pages)
    nat = pa.Scheduler(pool, slots, bs, max_blocks, chunk)
    ora = S.Scheduler(slots, bs, max_blocks, chunk, S.Pool(pages))
    next_id, steps = 0, 0
    pending = list(range(n_req))
    while steps < 20000:
        # arrivals between steps
        for _ in range(int(rng.integers(0, arrivals + 1)) if pending else 0):
            rid = pending.pop(0)
            p, m = int(rng.integers(1, 400)), int(rng.integers(1, 60))
            ok = ora.submit(rid, p, m)
            if ok:
                nat.submit(rid, p, m)
            else:
                with pytest.raises(pa.PagedAttnError):
                    nat.submit(rid, p, m)
            if not pending:
                break
        # an early finish now and then (a queued or an active request)
        if finishes and rng.random() < finishes:
            cand = [r.rid for r in ora.queue + ora.active]
            if cand:
                rid = int(rng.choice(cand))
                assert ora.finish(rid)
                nat.finish(rid)
        want = ora.step()
        got = nat.step()
        _same(got, want, max_blocks)
        assert pool.num_free() == len(ora.pool.free)
        assert nat.pending() == len(ora.queue) + len(ora.active)
        steps += 1
        if not pending and nat.pending() == 0:
            break
    assert not pending and nat.pending() == 0
    nat.close()
    assert pool.num_free() == pages
    return steps


@pytest.mark.parametrize("seed", range(8))
def test_native_scheduler_matches_the_oracle(seed):
    bs = 16 if seed % 2 == 0 else 32
    steps = _drive(seed, slots=[1, 3, 8, 64][seed % 4], bs=bs, max_blocks=32,
                   chunk=[16, 100, 512, 2048][seed % 4], pages=[40, 90, 300, 2000][seed % 4],
                   n_req=120, arrivals=[1, 2, 5, 30][seed % 4], finishes=0.05 * (seed % 3))
    assert steps > 10


def test_tight_pool_many_slots():
    # admission is bound by pages, not slots: requests wait in order for pages
    _drive(123, slots=32, bs=16, max_blocks=30, chunk=256, pages=31, n_req=60, arrivals=60,
           finishes=0.0)


def test_validation_and_errors():
    pool = pa.PagePool(8)
    with pytest.raises(pa.PagedAttnError):
        pa.Scheduler(pool, 0, 16, 4, 16)
    s = pa.Scheduler(pool, 2, 16, 4, 16)
    s.submit(1, 60, 5)                      # ceil(64/16) = 4 blocks: fits the table
    for bad in ((2, 60, 6), (1, 5, 5), (3, 0, 1), (4, 1, 0)):
        with pytest.raises(pa.PagedAttnError):
            s.submit(*bad)
    with pytest.raises(pa.PagedAttnError):
        s.finish(99)
    assert s.pending() == 1
    # another user drains the pool after admission: the step schedules nothing
    plan = s.step()
    assert plan.kind == pa.STEP_PREFILL and plan.ctx_lens.tolist() == [16]
    taken = pool.alloc(pool.num_free())
    with pytest.raises(pa.PagedAttnError) as e:
        s.step()
    assert e.value.status == -2
    pool.free(taken)
    plan = s.step()
    assert plan.kind == pa.STEP_PREFILL and plan.ctx_lens.tolist() == [32]
    s.close()
    assert pool.num_free() == 8

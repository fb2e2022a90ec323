"""Pins for the copy-on-write oracle (oracle/pages.py): against the pinned gather, the
identity, and closed cases.  CPU only."""

from __future__ import annotations

import numpy as np

import oracle as O
import workloads as W


def test_copy_reads_back_and_leaves_the_rest():
    case = W.custom_case([40, 21], [40, 21], block_size=16, kind="prefill", seed=81, slack=2.0)
    kp, vp = W.sentinel_pool(case), W.sentinel_pool(case)
    O.kv_append(kp, vp, case.k_new, case.v_new, case.block_tables, case.cu_new_lens,
                case.ctx_lens, 16)
    k0, v0 = kp.copy(), vp.copy()
    src = [int(case.block_tables[0][1]), int(case.block_tables[1][0])]
    used = set(case.block_tables[0][:3].tolist()) | set(case.block_tables[1][:2].tolist())
    free = [p for p in range(case.num_pages) if p not in used][:2]
    assert len(free) == 2
    O.copy_pages(kp, vp, src, free)
    for s, d in zip(src, free):
        assert np.array_equal(kp[d], k0[s]) and np.array_equal(vp[d], v0[s])
    other = [p for p in range(case.num_pages) if p not in free]
    assert np.array_equal(kp[other], k0[other]) and np.array_equal(vp[other], v0[other])


def test_remapped_block_table_gathers_the_same_kv():
    case = W.custom_case([70], [70], block_size=16, kind="prefill", seed=82, slack=2.0)
    kp, vp = W.sentinel_pool(case), W.sentinel_pool(case)
    O.kv_append(kp, vp, case.k_new, case.v_new, case.block_tables, case.cu_new_lens,
                case.ctx_lens, 16)
    bt = case.block_tables[0][:5].copy()
    free = [p for p in range(case.num_pages) if p not in set(bt.tolist())][:5]
    assert len(free) == 5
    O.copy_pages(kp, vp, bt, free)
    k1, v1 = O.gather(kp, vp, bt, 70, 16, 8, 64)
    k2, v2 = O.gather(kp, vp, np.array(free), 70, 16, 8, 64)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


def test_copy_onto_itself_and_bad_ids():
    case = W.custom_case([33], [33], block_size=32, kind="prefill", seed=83)
    kp, vp = W.sentinel_pool(case), W.sentinel_pool(case)
    O.kv_append(kp, vp, case.k_new, case.v_new, case.block_tables, case.cu_new_lens,
                case.ctx_lens, 32)
    k0, v0 = kp.copy(), vp.copy()
    p = int(case.block_tables[0][0])
    O.copy_pages(kp, vp, [p, -1, p], [p, p, case.num_pages])
    assert np.array_equal(kp, k0) and np.array_equal(vp, v0)


def test_cow_decisions_closed_cases():
    need, refs = O.cow_needs({3: 1, 5: 2, 7: 4}, [3, 5, 7])
    assert need == [False, True, True] and refs == {3: 1, 5: 1, 7: 3}
    # a page referenced by k sequences, each writing into it in turn: k - 1 copies, and the
    # last writer keeps the original
    refs = {9: 4}
    copies = 0
    for _ in range(4):
        need, refs = O.cow_needs(refs, [9])
        copies += need[0]
    assert copies == 3 and refs == {9: 1}
    # the same page twice in one list: decided entry by entry
    need, refs = O.cow_needs({4: 2}, [4, 4])
    assert need == [True, False] and refs == {4: 1}

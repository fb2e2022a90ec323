"""CPU oracle for page copy-on-write: page copies and which shared pages need one.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library and imports nothing from it.

Sources (cited by title and section):
  [guide]  "tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §PagedAttention：从操作系统借来的智慧:
           fixed-size pages reached through a block table make memory sharing, and with
           it copy-on-write, straightforward.
  [实战]   "Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎", §内存池管理: a preallocated
           pool and a free-page list; requests may share pages.

What is computed.  A page that more than one sequence references must not be written in
place: the writer first takes a fresh page, copies the shared page's K and V into it, and
points its own block-table entry at the copy, dropping one reference from the original.
A page with a single reference is written in place.

Readings taken where the pages are silent:
  * a copy moves the whole page (every KV head, every slot) of both pools, bit for bit;
  * the decision is taken per block-table entry, in order: an entry whose page has more
    than one reference at its turn gets a copy and lowers that count by one.

Parity pins (tests/test_oracle_pages.py): a copied page reads back bit-identical and every
other page is untouched; gathering a sequence through a block table remapped to the copies
gives the same K/V as through the originals; copying a page onto itself changes nothing;
closed cases of the per-entry decision (one reference: no copy; k references taken by k
writers in turn: k - 1 copies).
"""

from __future__ import annotations

from typing import Sequence

import numpy as np


def copy_pages(k_pool: np.ndarray, v_pool: np.ndarray, src: Sequence[int],
               dst: Sequence[int]) -> None:
    """Copy page src[i] onto page dst[i] in both pools (uint16 [num_pages, page_elems]),
    in place, in list order.  Pairs with an id outside the pool are skipped."""
    n = k_pool.shape[0]
    for s, d in zip(src, dst):
        s, d = int(s), int(d)
        if 0 <= s < n and 0 <= d < n:
            k_pool[d] = k_pool[s].copy()
            v_pool[d] = v_pool[s].copy()


def cow_needs(refcounts: dict, pages: Sequence[int]) -> tuple[list, dict]:
    """Per entry of ``pages`` (in order): whether it needs a private copy, and the
    reference counts of the original pages afterwards (fresh copies not included)."""
    refs = dict(refcounts)
    need = []
    for p in pages:
        if refs[p] > 1:
            need.append(True)
            refs[p] -= 1
        else:
            need.append(False)
    return need, refs

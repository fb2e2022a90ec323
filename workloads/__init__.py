"""Seeded synthetic inputs for paged KV attention at the Llama-3.2-1B attention shape.

Test infrastructure shared by the oracle tests, the GPU parity tests and ``bench.py``.
This module draws random numbers and lays out the integer bookkeeping of a batch
(sequence lengths, which physical page backs which logical block, block tables).
It performs none of the attention arithmetic and knows nothing about how tokens are
arranged inside a page: each side (the CPU oracle and the HIP library) writes the
logical K/V rows produced here into its own pools with its own ``kv_append``.

Workloads (the five shapes the hot path is measured on; 32 query heads, 8 KV heads,
head_dim 64, bf16 values, scale 1/8):

1. single-sequence decode: 1 sequence, context 37, block size 16, pool of 64 pages,
   block table = seeded distinct random page ids.
2. batched decode: 64 sequences, context uniform in [1, 2048], block size 16, pool =
   needed pages + 10 %, shuffled page assignment.
3. prefill: 8 prompts, length uniform in [128, 1024], block size 16, K/V appended into
   shuffled pages, then causal attention over them.
4. long-context decode: 16 sequences of context 32768, block size 32, K/V ~ N(0, 0.5^2).
5. mixed continuous-batch step (per layer, 16 layers): a 512-token prefill chunk whose
   first 512 prompt tokens are already cached, plus 128 decode sequences with context
   uniform in [16, 8192]; the first 256 tokens of 32 decode sequences share pages.

Every random draw comes from ``numpy.random.default_rng(SeedSequence([31, cfg, layer,
stream, block]))`` with streams 0 = lengths, 1 = page assignment, 2 = Q, 3 = K, 4 = V.
Floats are ``standard_normal(float32) * sigma`` rounded to bfloat16 (round to nearest
even) here on the host, so the bytes do not depend on the machine.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

ROOT_SEED = 31
SENTINEL_BITS = 0x7FDA  # a quiet-NaN bfloat16 pattern; fills every pool byte no append wrote
_BLOCK = 1 << 22  # values per independently seeded block of a float stream


# ---------------------------------------------------------------------------------------
# random bf16 streams
# ---------------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values (finite) to bfloat16 bit patterns, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal_block(words: Sequence[int], n: int, sigma: float) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(list(words)))
    x = rng.standard_normal(n, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def normal_bf16(words: Sequence[int], n: int, sigma: float = 1.0) -> np.ndarray:
    """``n`` bf16 draws of N(0, sigma^2); block b of the stream is seeded by words+[b].

    The split into fixed blocks makes the bytes independent of how many threads fill them.
    """
    out = np.empty(n, dtype=np.uint16)
    nblk = (n + _BLOCK - 1) // _BLOCK
    if nblk <= 1:
        if n:
            out[:] = _normal_block(list(words) + [0], n, sigma)
        return out

    def fill(b: int) -> None:
        lo = b * _BLOCK
        hi = min(n, lo + _BLOCK)
        out[lo:hi] = _normal_block(list(words) + [b], hi - lo, sigma)

    workers = max(1, min(16, len(os.sched_getaffinity(0)), nblk))
    with _cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def _rng(cfg: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, cfg, layer, stream]))


# ---------------------------------------------------------------------------------------
# a batch
# ---------------------------------------------------------------------------------------
@dataclasses.dataclass
class Case:
    """One batch of the hot path: integer structure plus one layer's bf16 values.

    Sequence ``s`` holds ``ctx_lens[s]`` tokens once the step's append has run.  Before
    the step, positions ``[setup_start[s], ctx_lens[s] - new_lens[s])`` are appended by a
    setup call (positions below ``setup_start[s]`` live on pages another sequence wrote:
    shared prefix pages).  The step appends ``new_lens[s]`` tokens at positions
    ``[ctx_lens[s] - new_lens[s], ctx_lens[s])``.

    ``decode_seqs`` / ``prefill_seqs`` are contiguous index ranges.  A decode sequence
    has exactly one query row (its newest token); a prefill sequence has one query row
    per appended token.  All float arrays are raw bf16 bit patterns (uint16).
    """

    name: str
    cfg: int
    layer: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_pages: int
    scale: float
    ctx_lens: np.ndarray  # int32 [n]
    new_lens: np.ndarray  # int32 [n]
    setup_start: np.ndarray  # int32 [n]
    block_tables: np.ndarray  # int32 [n, max_blocks]
    sentinel_page: int  # an unassigned page; fills unused block-table entries
    decode_seqs: range
    prefill_seqs: range
    shared_seqs: np.ndarray  # int32, sequences whose first pages are shared (may be empty)
    shared_prefix_tokens: int
    sigma_q: float
    sigma_kv: float
    # per-layer values
    q_decode: Optional[np.ndarray] = None  # uint16 [len(decode_seqs), Hq, d]
    q_prefill: Optional[np.ndarray] = None  # uint16 [sum new_lens over prefill seqs, Hq, d]
    k_new: Optional[np.ndarray] = None  # uint16 [sum new_lens, Hkv, d]
    v_new: Optional[np.ndarray] = None
    k_setup: Optional[np.ndarray] = None  # uint16 [sum setup lens, Hkv, d]
    v_setup: Optional[np.ndarray] = None

    # ---- derived integer views -------------------------------------------------------
    @property
    def n_seqs(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def cu_new_lens(self) -> np.ndarray:
        return _cumsum0(self.new_lens)

    @property
    def setup_ctx_lens(self) -> np.ndarray:
        return (self.ctx_lens - self.new_lens).astype(np.int32)

    @property
    def setup_new_lens(self) -> np.ndarray:
        return (self.setup_ctx_lens - self.setup_start).astype(np.int32)

    @property
    def cu_setup_lens(self) -> np.ndarray:
        return _cumsum0(self.setup_new_lens)

    @property
    def q_lens_prefill(self) -> np.ndarray:
        return self.new_lens[self.prefill_seqs.start:self.prefill_seqs.stop].astype(np.int32)

    @property
    def cu_q_lens_prefill(self) -> np.ndarray:
        return _cumsum0(self.q_lens_prefill)

    def kv_tokens(self) -> int:
        """Logical context tokens read by the decode sequences (one layer)."""
        d = self.ctx_lens[self.decode_seqs.start:self.decode_seqs.stop]
        return int(d.astype(np.int64).sum())

    def prefill_pairs(self, causal: bool = True) -> int:
        """Visible (query, key) pairs of the prefill sequences (one layer, one q head)."""
        tot = 0
        for s in self.prefill_seqs:
            ctx = int(self.ctx_lens[s])
            ql = int(self.new_lens[s])
            if causal:
                base = ctx - ql
                tot += ql * base + ql * (ql + 1) // 2
            else:
                tot += ql * ctx
        return tot

    def logical_kv(self, s: int):
        """Logical K and V rows [ctx, Hkv, d] (bf16 bits) of sequence ``s``, in position
        order, reassembled from the setup and step arrays (integer bookkeeping only)."""
        assert self.k_new is not None and self.k_setup is not None
        ctx = int(self.ctx_lens[s])
        start = int(self.setup_start[s])
        parts_k, parts_v = [], []
        if start > 0:
            lead = int(self.shared_seqs[0])
            lk, lv = self.logical_kv(lead)
            parts_k.append(lk[:start])
            parts_v.append(lv[:start])
        a, b = self.cu_setup_lens[s], self.cu_setup_lens[s + 1]
        parts_k.append(self.k_setup[a:b])
        parts_v.append(self.v_setup[a:b])
        a, b = self.cu_new_lens[s], self.cu_new_lens[s + 1]
        parts_k.append(self.k_new[a:b])
        parts_v.append(self.v_new[a:b])
        k = np.concatenate(parts_k, axis=0)
        v = np.concatenate(parts_v, axis=0)
        assert k.shape[0] == ctx
        return k, v


def _cumsum0(x: np.ndarray) -> np.ndarray:
    out = np.zeros(len(x) + 1, dtype=np.int32)
    np.cumsum(x, out=out[1:])
    return out


def _assign_pages(ctx_lens, block_size, num_pages, perm, shared_seqs=(), shared_blocks=0):
    """Consume ``perm`` in (sequence, logical block) order.  Sequences in ``shared_seqs``
    after the first reuse the first ``shared_blocks`` pages of the first one."""
    n = len(ctx_lens)
    max_blocks = max(1, max((int(c) + block_size - 1) // block_size for c in ctx_lens))
    bt = np.full((n, max_blocks), -1, dtype=np.int64)
    k = 0
    shared = list(shared_seqs)
    lead = shared[0] if shared else -1
    for s in range(n):
        nb = (int(ctx_lens[s]) + block_size - 1) // block_size
        for b in range(nb):
            if s in shared and s != lead and b < shared_blocks:
                bt[s, b] = bt[lead, b]
            else:
                bt[s, b] = perm[k]
                k += 1
    assert k < num_pages, "pool must keep at least one unassigned page"
    sentinel = int(perm[k])
    bt[bt < 0] = sentinel
    return bt.astype(np.int32), sentinel, k


def pool_pages_for(needed: int, slack: float = 0.10) -> int:
    """Pool size: needed pages plus ``slack`` (rounded up), and never zero slack pages."""
    return max(needed + 1, int(math.ceil(needed * (1.0 + slack))))


def build_case(
    *,
    name: str,
    cfg: int,
    ctx_lens: Sequence[int],
    new_lens: Sequence[int],
    block_size: int,
    decode_seqs: range,
    prefill_seqs: range,
    num_q_heads: int = 32,
    num_kv_heads: int = 8,
    head_dim: int = 64,
    num_pages: Optional[int] = None,
    perm: Optional[np.ndarray] = None,
    shared_seqs: Sequence[int] = (),
    shared_prefix_tokens: int = 0,
    sigma_q: float = 1.0,
    sigma_kv: float = 1.0,
    scale: Optional[float] = None,
    layer: int = 0,
    values: bool = True,
) -> Case:
    """Integer structure for a batch, then (``values=True``) one layer's bf16 values."""
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    new = np.asarray(new_lens, dtype=np.int32)
    assert ctx.shape == new.shape and np.all(new <= ctx) and np.all(new >= 0)
    for s in decode_seqs:
        assert new[s] <= 1, "a decode sequence appends at most one token"
    shared = np.asarray(list(shared_seqs), dtype=np.int32)
    assert shared_prefix_tokens % block_size == 0
    shared_blocks = shared_prefix_tokens // block_size
    for s in shared:
        assert ctx[s] - new[s] >= shared_prefix_tokens, "shared pages must be full and cached"
    needed = int(sum((int(c) + block_size - 1) // block_size for c in ctx))
    if len(shared):
        needed -= (len(shared) - 1) * shared_blocks
    if num_pages is None:
        num_pages = pool_pages_for(needed)
    if perm is None:
        perm = _rng(cfg, 0, 1).permutation(num_pages)
    bt, sentinel, _ = _assign_pages(ctx, block_size, num_pages, perm, shared, shared_blocks)
    setup_start = np.zeros_like(ctx)
    if len(shared):
        setup_start[shared[1:]] = shared_prefix_tokens
    case = Case(
        name=name, cfg=cfg, layer=layer,
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        block_size=block_size, num_pages=int(num_pages),
        scale=(1.0 / math.sqrt(head_dim)) if scale is None else float(scale),
        ctx_lens=ctx, new_lens=new, setup_start=setup_start,
        block_tables=bt, sentinel_page=sentinel,
        decode_seqs=decode_seqs, prefill_seqs=prefill_seqs,
        shared_seqs=shared, shared_prefix_tokens=int(shared_prefix_tokens),
        sigma_q=sigma_q, sigma_kv=sigma_kv,
    )
    if values:
        fill_values(case, layer)
    return case


def fill_values(case: Case, layer: int) -> Case:
    """Draw one layer's Q, K and V (streams 2, 3, 4) into ``case``."""
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    n_dec = len(case.decode_seqs)
    tq = int(case.q_lens_prefill.sum())
    t_new = int(case.new_lens.sum())
    t_setup = int(case.setup_new_lens.sum())
    c = case.cfg
    case.layer = layer
    q = normal_bf16([ROOT_SEED, c, layer, 2], (n_dec + tq) * hq * d, case.sigma_q)
    case.q_decode = q[: n_dec * hq * d].reshape(n_dec, hq, d)
    case.q_prefill = q[n_dec * hq * d:].reshape(tq, hq, d)
    k = normal_bf16([ROOT_SEED, c, layer, 3], (t_setup + t_new) * hkv * d, case.sigma_kv)
    v = normal_bf16([ROOT_SEED, c, layer, 4], (t_setup + t_new) * hkv * d, case.sigma_kv)
    case.k_setup = k[: t_setup * hkv * d].reshape(t_setup, hkv, d)
    case.k_new = k[t_setup * hkv * d:].reshape(t_new, hkv, d)
    case.v_setup = v[: t_setup * hkv * d].reshape(t_setup, hkv, d)
    case.v_new = v[t_setup * hkv * d:].reshape(t_new, hkv, d)
    return case


# ---------------------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "decode-1seq-ctx37-bs16",
    2: "decode-64seq-ctx1..2048-bs16",
    3: "prefill-8prompts-128..1024-bs16",
    4: "decode-16seq-ctx32768-bs32-splitk",
    5: "mixed-step-16layer-chunk512-128decode-bs32",
}
NUM_LAYERS = {1: 1, 2: 1, 3: 1, 4: 1, 5: 16}


def make_case(cfg: int, layer: int = 0, values: bool = True) -> Case:
    """The integer structure of workload ``cfg`` (identical for every layer) plus, when
    ``values`` is set, the bf16 values of layer ``layer``."""
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        perm = _rng(1, 0, 1).permutation(64)
        return build_case(name=name, cfg=1, ctx_lens=[37], new_lens=[1], block_size=16,
                          num_pages=64, perm=perm, decode_seqs=range(0, 1),
                          prefill_seqs=range(1, 1), layer=layer, values=values)
    if cfg == 2:
        ctx = _rng(2, 0, 0).integers(1, 2048, size=64, endpoint=True)
        return build_case(name=name, cfg=2, ctx_lens=ctx, new_lens=np.ones(64, np.int32),
                          block_size=16, decode_seqs=range(0, 64), prefill_seqs=range(64, 64),
                          layer=layer, values=values)
    if cfg == 3:
        # stratified uniform draw: each length is uniform on [128, 1024] and the eight
        # fall in distinct eighths of the range, so the total stays near 8 x 576 = 4.6k
        r = _rng(3, 0, 0)
        strata = r.permutation(8)
        u = r.random(8)
        lens = 128 + np.floor((strata + u) * (897 / 8)).astype(np.int64)
        return build_case(name=name, cfg=3, ctx_lens=lens, new_lens=lens, block_size=16,
                          decode_seqs=range(0, 0), prefill_seqs=range(0, 8),
                          layer=layer, values=values)
    if cfg == 4:
        ctx = np.full(16, 32768, np.int32)
        return build_case(name=name, cfg=4, ctx_lens=ctx, new_lens=np.ones(16, np.int32),
                          block_size=32, decode_seqs=range(0, 16), prefill_seqs=range(16, 16),
                          sigma_kv=0.5, layer=layer, values=values)
    if cfg == 5:
        n_dec = 128
        dec_ctx = _rng(5, 0, 0).integers(16, 8192, size=n_dec, endpoint=True)
        eligible = [s for s in range(n_dec) if dec_ctx[s] >= 257]
        assert len(eligible) >= 32
        shared = eligible[:32]
        ctx = np.concatenate([dec_ctx, [1024]]).astype(np.int32)
        new = np.concatenate([np.ones(n_dec, np.int32), [512]]).astype(np.int32)
        return build_case(name=name, cfg=5, ctx_lens=ctx, new_lens=new, block_size=32,
                          decode_seqs=range(0, n_dec), prefill_seqs=range(n_dec, n_dec + 1),
                          shared_seqs=shared, shared_prefix_tokens=256,
                          layer=layer, values=values)
    raise ValueError(f"unknown workload {cfg}")


def custom_case(
    ctx_lens: Sequence[int],
    new_lens: Sequence[int],
    *,
    block_size: int = 16,
    kind: str = "decode",
    num_q_heads: int = 32,
    num_kv_heads: int = 8,
    head_dim: int = 64,
    seed: int = 0,
    sigma_q: float = 1.0,
    sigma_kv: float = 1.0,
    shared_seqs: Sequence[int] = (),
    shared_prefix_tokens: int = 0,
    slack: float = 0.10,
) -> Case:
    """A small batch for tests: ``kind`` is 'decode' (every sequence served by the decode
    call) or 'prefill' (every sequence served by the prefill call).  ``seed`` picks an
    independent family of streams (it takes the place of the workload number)."""
    n = len(ctx_lens)
    cfg = 1000 + int(seed)
    if kind == "decode":
        dec, pre = range(0, n), range(n, n)
    elif kind == "prefill":
        dec, pre = range(0, 0), range(0, n)
    else:
        raise ValueError(kind)
    needed = sum((int(c) + block_size - 1) // block_size for c in ctx_lens)
    if shared_seqs:
        needed -= (len(shared_seqs) - 1) * (shared_prefix_tokens // block_size)
    num_pages = pool_pages_for(needed, slack)
    return build_case(name=f"custom-{seed}", cfg=cfg, ctx_lens=ctx_lens, new_lens=new_lens,
                      block_size=block_size, decode_seqs=dec, prefill_seqs=pre,
                      num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                      num_pages=num_pages, shared_seqs=shared_seqs,
                      shared_prefix_tokens=shared_prefix_tokens,
                      sigma_q=sigma_q, sigma_kv=sigma_kv)


def page_elems(case: Case) -> int:
    """bf16 values held by one page of one pool (K or V) of one layer."""
    return case.block_size * case.num_kv_heads * case.head_dim


def sentinel_pool(case: Case) -> np.ndarray:
    """A pool (one of K, V) filled with the NaN sentinel, as flat bf16 bits per page."""
    return np.full((case.num_pages, page_elems(case)), SENTINEL_BITS, dtype=np.uint16)

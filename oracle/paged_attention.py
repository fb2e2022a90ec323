"""CPU oracle for paged KV attention: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (``paged_kv_attention_31_amd``)
and imports nothing from it.

Sources (cited by title and section):
  [guide]  "tiny-vllm：从零构建高性能LLM推理引擎的完整指南" (zingnex.cn)
  [实战]   "Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎" (blog.hotdry.top)

What the method computes.  Paging moves where K/V bytes live, not the result
([guide] §PagedAttention: the cache is cut into fixed-size blocks reached through a
block table).  Online softmax and tiling are exact rewrites of the three-pass softmax
([实战] §算子融合; [guide] §在线Softmax).  So the oracle is the plain definition:
gather the pages back into contiguous K/V, then causal grouped-query softmax attention
([guide] §Llama 3.2 1B架构拆解: GQA, causal mask, softmax, weighted sum of V), with
the new token's K/V appended before it attends ([guide] §推理流程：从Prefill到Decode).

Readings taken where the pages are silent:
  * query head h reads KV head h // (Hq / Hkv) (contiguous groups);
  * scores are scaled by ``scale`` (1/sqrt(64) = 1/8) before the max;
  * a query at absolute position p sees keys 0..p inclusive (bottom-right causal);
    a decode row sits at position ctx-1, so ``ctx_len`` counts the appended token;
  * a row that sees no key returns zeros;
  * page layout: separate K and V pools of ``[num_pages][page]`` bf16; inside one page
    K is ``[Hkv][d/8][bs][8]`` (16-byte pieces of a token's head vector, grouped by
    piece) and V is ``[Hkv][d][bs]`` (one row per dimension).  The pages fix only what
    a page holds (block_size x head_dim x num_kv_heads values, [实战] §内存池管理), not
    the order; the order appears in ``k_offset`` / ``v_offset`` and nowhere else here.

Parity pins (tests/test_oracle.py): brute-force dense attention on tiny inputs;
page-permutation invariance; one-pass online softmax and the split-K merge against the
three-pass result; context 1 returns V; q = 0 returns the mean of V; linearity in V;
shared prefix pages; chunked == one-shot prefill; last prefill row == decode; GQA head
groups; append/gather round trip; the 16 KB page of [实战] §内存池管理.
"""

from __future__ import annotations

import math
from typing import Sequence

import numpy as np

# ---------------------------------------------------------------------------------------
# bf16 ([guide] §BF16浮点数: 1 sign, 8 exponent, 7 mantissa bits -- the top half of fp32)
# ---------------------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns exactly: a bf16 value is the fp32 value whose top 16 bits
    are the pattern and whose low 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def page_bytes(block_size: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Bytes of one page of one pool (K or V) of one layer ([实战] §内存池管理: a page holds
    page_size x head_dim x num_kv_heads bf16 values)."""
    return block_size * head_dim * num_kv_heads * elem_bytes


# ---------------------------------------------------------------------------------------
# page layout (the only place it appears in the oracle)
# ---------------------------------------------------------------------------------------


def k_offset(g: int, slot: int, i: int, block_size: int, head_dim: int) -> int:
    """Element offset inside a K page of token ``slot``, KV head ``g``, dimension ``i``:
    layout [Hkv][head_dim/8][block_size][8]."""
    return ((g * (head_dim // 8) + i // 8) * block_size + slot) * 8 + (i % 8)


def v_offset(g: int, slot: int, i: int, block_size: int, head_dim: int) -> int:
    """Element offset inside a V page: layout [Hkv][head_dim][block_size]."""
    return (g * head_dim + i) * block_size + slot


def _token_offsets(block_size: int, num_kv_heads: int, head_dim: int, slot: int):
    ko = np.empty((num_kv_heads, head_dim), dtype=np.int64)
    vo = np.empty((num_kv_heads, head_dim), dtype=np.int64)
    for g in range(num_kv_heads):
        for i in range(head_dim):
            ko[g, i] = k_offset(g, slot, i, block_size, head_dim)
            vo[g, i] = v_offset(g, slot, i, block_size, head_dim)
    return ko, vo


class _Offsets:
    """Per-slot offset tables, built once per geometry from k_offset / v_offset."""

    _cache: dict = {}

    @classmethod
    def get(cls, block_size: int, num_kv_heads: int, head_dim: int):
        key = (block_size, num_kv_heads, head_dim)
        if key not in cls._cache:
            ks, vs = zip(*(_token_offsets(block_size, num_kv_heads, head_dim, s)
                           for s in range(block_size)))
            cls._cache[key] = (np.stack(ks), np.stack(vs))  # [bs][Hkv][d]
        return cls._cache[key]


# ---------------------------------------------------------------------------------------
# kv_append and gather ([guide] §推理流程: each new token's K/V is appended to the cache
# before attention; [guide] §PagedAttention: logical block -> physical block via the
# block table)
# ---------------------------------------------------------------------------------------


def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              block_tables: np.ndarray, cu_new_lens: np.ndarray, ctx_lens: np.ndarray,
              block_size: int) -> None:
    """Copy new token rows into the pools, in place (bit copy, no rounding).

    ``k_pool``/``v_pool``: uint16 [num_pages, page_elems].  ``k_new``/``v_new``: uint16
    [T, Hkv, d].  Token j of sequence s (``cu_new_lens[s] <= j < cu_new_lens[s+1]``) sits
    at position ``ctx_lens[s] - n_s + (j - cu_new_lens[s])``, i.e. in page
    ``block_tables[s][pos // block_size]`` at slot ``pos % block_size``.
    """
    _, hkv, d = k_new.shape
    ko, vo = _Offsets.get(block_size, hkv, d)
    n = len(ctx_lens)
    for s in range(n):
        a, b = int(cu_new_lens[s]), int(cu_new_lens[s + 1])
        first = int(ctx_lens[s]) - (b - a)
        for j in range(a, b):
            pos = first + (j - a)
            page = int(block_tables[s][pos // block_size])
            slot = pos % block_size
            k_pool[page][ko[slot].ravel()] = k_new[j].ravel()
            v_pool[page][vo[slot].ravel()] = v_new[j].ravel()


def gather(k_pool: np.ndarray, v_pool: np.ndarray, block_table: Sequence[int], ctx: int,
           block_size: int, num_kv_heads: int, head_dim: int):
    """Logical K, V of one sequence as uint16 [ctx, Hkv, d] (bits), position order."""
    ko, vo = _Offsets.get(block_size, num_kv_heads, head_dim)
    k = np.empty((ctx, num_kv_heads, head_dim), dtype=np.uint16)
    v = np.empty((ctx, num_kv_heads, head_dim), dtype=np.uint16)
    for p in range(ctx):
        page = int(block_table[p // block_size])
        slot = p % block_size
        k[p] = k_pool[page][ko[slot]]
        v[p] = v_pool[page][vo[slot]]
    return k, v


# ---------------------------------------------------------------------------------------
# attention, three-pass softmax ([实战] §算子融合: max, then sum of exponentials, then
# normalise), grouped-query heads ([guide] §Llama 3.2 1B架构拆解)
# ---------------------------------------------------------------------------------------


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_visible: Sequence[int],
              scale: float) -> np.ndarray:
    """Softmax attention of query rows over one sequence's contiguous K/V, in fp64.

    ``q``: float64 [R, Hq, d]; ``k``, ``v``: float64 [T, Hkv, d]; row r sees keys
    ``0 .. n_visible[r]-1``.  Returns float64 [R, Hq, d]; a row that sees nothing is 0.
    """
    r_rows, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.zeros((r_rows, hq, d), dtype=np.float64)
    for r in range(r_rows):
        n = int(n_visible[r])
        if n <= 0:
            continue
        for h in range(hq):
            g = h // group
            x = scale * (k[:n, g, :] @ q[r, h, :])  # scores, [n]
            m = np.max(x)  # pass 1: maximum
            w = np.exp(x - m)  # pass 2: exponentials and their sum
            den = np.sum(w)
            out[r, h, :] = (w / den) @ v[:n, g, :]  # pass 3: normalise, weight V
    return out


def online_softmax_attention(q_row: np.ndarray, k: np.ndarray, v: np.ndarray, n: int,
                             scale: float) -> np.ndarray:
    """One row, one pass over keys, keeping a running maximum and a running sum that is
    rescaled whenever the maximum grows ([实战] §算子融合; [guide] §在线Softmax).
    ``q_row``: [Hq, d]; returns [Hq, d] float64."""
    hq, d = q_row.shape
    group = hq // k.shape[1]
    out = np.zeros((hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // group
        m = -math.inf
        den = 0.0
        acc = np.zeros(d, dtype=np.float64)
        for t in range(n):
            x = scale * float(k[t, g, :] @ q_row[h, :])
            m_new = max(m, x)
            c = math.exp(m - m_new) if m != -math.inf else 0.0
            p = math.exp(x - m_new)
            den = den * c + p
            acc = acc * c + p * v[t, g, :]
            m = m_new
        if n > 0:
            out[h] = acc / den
    return out


def partition_partials(q_row: np.ndarray, k: np.ndarray, v: np.ndarray, n: int, scale: float,
                       part: int):
    """Split keys 0..n-1 into chunks of ``part`` and return, per chunk j and head h, the
    chunk maximum m, the chunk sum l = sum exp(x - m) and o = sum exp(x - m) v
    (unnormalised).  An empty chunk has m = -inf, l = 0, o = 0."""
    hq, d = q_row.shape
    group = hq // k.shape[1]
    n_parts = max(1, (n + part - 1) // part)
    m = np.full((n_parts, hq), -np.inf)
    den = np.zeros((n_parts, hq))
    o = np.zeros((n_parts, hq, d))
    for j in range(n_parts):
        lo, hi = j * part, min(n, (j + 1) * part)
        if hi <= lo:
            continue
        for h in range(hq):
            g = h // group
            x = scale * (k[lo:hi, g, :] @ q_row[h, :])
            m[j, h] = np.max(x)
            w = np.exp(x - m[j, h])
            den[j, h] = np.sum(w)
            o[j, h] = w @ v[lo:hi, g, :]
    return m, den, o


def merge_partials(m: np.ndarray, den: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Log-sum-exp merge of chunk partials: M = max_j m_j, L = sum_j l_j e^(m_j - M),
    out = sum_j o_j e^(m_j - M) / L.  Chunks with m = -inf are skipped; a row with no
    chunk returns 0.  Shapes: m, den [P, Hq]; o [P, Hq, d] -> [Hq, d]."""
    n_parts, hq, d = o.shape
    out = np.zeros((hq, d))
    for h in range(hq):
        live = [j for j in range(n_parts) if m[j, h] != -np.inf]
        if not live:
            continue
        big = max(m[j, h] for j in live)
        num = np.zeros(d)
        tot = 0.0
        for j in live:
            f = math.exp(m[j, h] - big)
            tot += den[j, h] * f
            num += o[j, h] * f
        out[h] = num / tot
    return out


# ---------------------------------------------------------------------------------------
# the two phases ([guide] §推理流程：从Prefill到Decode)
# ---------------------------------------------------------------------------------------


def decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
           ctx_lens: Sequence[int], block_size: int, num_kv_heads: int, head_dim: int,
           scale: float, seqs: Sequence[int] | None = None) -> np.ndarray:
    """Decode: one query row per sequence, at position ctx-1, seeing all ctx keys.

    ``q``: bf16 bits [n, Hq, d]; pools: bits [P, page]; returns float64 [n, Hq, d]
    (rows not listed in ``seqs`` stay 0)."""
    n, hq, d = q.shape
    out = np.zeros((n, hq, d), dtype=np.float64)
    for s in (range(n) if seqs is None else seqs):
        ctx = int(ctx_lens[s])
        kb, vb = gather(k_pool, v_pool, block_tables[s], ctx, block_size, num_kv_heads, head_dim)
        out[s] = attention(bf16_to_f64(q[s:s + 1]), bf16_to_f64(kb), bf16_to_f64(vb),
                           [ctx], scale)[0]
    return out


def prefill(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
            cu_q_lens: Sequence[int], ctx_lens: Sequence[int], block_size: int,
            num_kv_heads: int, head_dim: int, scale: float, causal: bool = True) -> np.ndarray:
    """Prefill (or a prefill chunk): query row i of sequence s sits at position
    ctx - qlen + i and sees keys 0..pos (causal) or all ctx keys (non-causal).

    ``q``: bf16 bits [Tq, Hq, d] packed by ``cu_q_lens``; returns float64 [Tq, Hq, d]."""
    tq, hq, d = q.shape
    out = np.zeros((tq, hq, d), dtype=np.float64)
    for s in range(len(ctx_lens)):
        a, b = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        if b <= a:
            continue
        ctx = int(ctx_lens[s])
        qlen = b - a
        kb, vb = gather(k_pool, v_pool, block_tables[s], ctx, block_size, num_kv_heads, head_dim)
        vis = [(ctx - qlen + i + 1) if causal else ctx for i in range(qlen)]
        out[a:b] = attention(bf16_to_f64(q[a:b]), bf16_to_f64(kb), bf16_to_f64(vb), vis, scale)
    return out

"""CPU oracle for rotary position encoding fused into the K/V append: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library and imports nothing from it.

Sources (cited by title and section):
  [guide]  "tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §Llama 3.2 1B架构拆解: the
           attention sub-layer applies rotary position encoding to Q and K, injecting each
           token's position before attention; §推理流程：从Prefill到Decode: a token's K/V
           joins the cache before the token attends.
  [实战]   "Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎" (introduction): RoPE is one
           of the engine's hand-written kernels.

What is computed.  Each head vector is split into d/2 coordinate pairs and pair i is
turned through the angle p * f_i, where p is the token's absolute position in its
sequence.  The rotated K joins the page cache exactly where the plain append would put
it; V is copied unchanged; Q is rotated with the same positions and returned.

Readings taken where the pages are silent:
  * pair i is (x[i], x[i + d/2]) ("rotate half"), turned counter-clockwise:
    (a, b) -> (a cos t - b sin t, b cos t + a sin t);
  * f_i = theta ** (-2 i / d) with a caller-given base theta (500000 for the Llama 3
    family), or a caller-given table of d/2 frequencies (any rescaled variant);
  * position p of new token j of sequence s is ctx_lens[s] - n_s + j, as for the append;
  * the rotation is done in fp64 on the bf16 inputs and rounded once to bf16, to nearest
    with ties to even.

Parity pins (tests/test_oracle_rope.py): position 0 is the identity, bit for bit; the
rotation equals complex multiplication by exp(i t) (numpy complex128); pair norms are
kept; q.k after rotation depends only on the position difference; the fp64 -> bf16
rounding against a brute-force nearest-value search; the fused append against the plain
append of the rotated rows; the frequency table's closed-form ratios.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .paged_attention import bf16_to_f64, kv_append


def rope_freqs(head_dim: int, theta: float) -> np.ndarray:
    """f_i = theta ** (-2 i / head_dim), i = 0 .. head_dim/2 - 1, in fp64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / head_dim)


def rotate(x: np.ndarray, pos: np.ndarray, freqs: np.ndarray) -> np.ndarray:
    """Rotate fp64 head vectors ``x[..., d]`` at positions ``pos`` (broadcast over the
    leading axes of x): pair i = (x[i], x[i + d/2]) turns by pos * freqs[i]."""
    x = np.asarray(x, dtype=np.float64)
    half = x.shape[-1] // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * np.asarray(freqs, dtype=np.float64)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 bit patterns, to nearest with ties to even, in one
    rounding: first to fp32 with round-to-odd (truncate, then set the last bit when
    anything was dropped), which keeps every tie of the final step a true tie, then from
    fp32 to bf16 by nearest-even on the top 16 bits.  Finite inputs only."""
    x = np.asarray(x, dtype=np.float64)
    y = x.astype(np.float32)  # nearest
    over = np.abs(y.astype(np.float64)) > np.abs(x)
    y = np.where(over, np.nextafter(y, np.float32(0)), y)  # now truncated toward zero
    bits = y.view(np.uint32).copy()
    inexact = y.astype(np.float64) != x
    bits |= inexact.astype(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def positions(cu_new_lens: np.ndarray, ctx_lens: np.ndarray) -> np.ndarray:
    """Absolute position of every new row: row j of sequence s (cu_new_lens[s] <= j <
    cu_new_lens[s+1]) sits at ctx_lens[s] - n_s + (j - cu_new_lens[s])."""
    n = len(ctx_lens)
    out = np.empty(int(cu_new_lens[n]), dtype=np.int64)
    for s in range(n):
        a, b = int(cu_new_lens[s]), int(cu_new_lens[s + 1])
        out[a:b] = int(ctx_lens[s]) - (b - a) + np.arange(b - a)
    return out


def rope_kv_append(q: Optional[np.ndarray], k_new: np.ndarray, v_new: np.ndarray,
                   k_pool: np.ndarray, v_pool: np.ndarray, block_tables: np.ndarray,
                   cu_new_lens: np.ndarray, ctx_lens: np.ndarray, block_size: int,
                   freqs: np.ndarray) -> Optional[np.ndarray]:
    """Rotate the new K rows (uint16 bf16 bits [T, Hkv, d]) and append them with V to the
    pools in place; return the rotated Q rows ([T, Hq, d] bits), or None without q."""
    pos = positions(cu_new_lens, ctx_lens)
    k_rot = f64_to_bf16(rotate(bf16_to_f64(k_new), pos[:, None], freqs))
    kv_append(k_pool, v_pool, k_rot, v_new, block_tables, cu_new_lens, ctx_lens, block_size)
    if q is None:
        return None
    return f64_to_bf16(rotate(bf16_to_f64(q), pos[:, None], freqs))

"""Shared test plumbing: build the oracle's pools for a generated batch and run the
oracle over a batch's decode and prefill sequences.  Test infrastructure only."""

from __future__ import annotations

import struct

import numpy as np

import oracle as O
import workloads as W


# The parity bar: max-abs 1e-2 and mean-abs 1e-3 of the bf16 output widened to fp32
# against the fp64 oracle rounded to fp32, over all elements of a case.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
# At |o| >= 4 two neighbouring bf16 values lie 2^-5 apart, so even the correctly rounded
# output can miss the exact value by 2^-6 > MAX_ABS.  Such elements are held to half a
# bf16 unit of the exact value plus R13_SLACK (the kernels' fp32 arithmetic can put a
# value within that of a rounding midpoint on the other side) and are counted.
R13_ABS = 4.0
R13_SLACK = 1e-3


def bf16_half_unit(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values around |x| (8 significant bits): 2^(e - 8) for
    |x| in [2^e, 2^(e+1))."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(ax)) - 8).astype(np.int64))


def parity_stats(gpu_f32: np.ndarray, ref_f64: np.ndarray) -> dict:
    """Element-wise comparison at the parity bar.  Returns max-abs and mean-abs over all
    elements, the counts of elements with |oracle| >= 2 and >= R13_ABS, the largest error
    among elements below R13_ABS, and whether every element meets its bar (MAX_ABS below
    R13_ABS, half a bf16 unit + R13_SLACK at or above it) and mean-abs <= MEAN_ABS."""
    g = np.asarray(gpu_f32, dtype=np.float32).reshape(-1)
    r = np.asarray(ref_f64, dtype=np.float64).astype(np.float32).reshape(-1)
    diff = np.abs(g.astype(np.float64) - r.astype(np.float64))
    big = np.abs(r) >= R13_ABS
    bar = np.where(big, bf16_half_unit(r) + R13_SLACK, MAX_ABS)
    excess = diff - bar
    n = diff.size
    st = {
        "n": int(n),
        "finite": bool(np.isfinite(g).all()),
        "max_abs": float(diff.max()) if n else 0.0,
        "mean_abs": float(diff.mean()) if n else 0.0,
        "max_abs_below_r13": float(diff[~big].max()) if (~big).any() else 0.0,
        "n_abs_ge_2": int((np.abs(r) >= 2.0).sum()),
        "n_abs_ge_4": int(big.sum()),
        "n_r13_over_max_abs": int((diff[big] > MAX_ABS).sum()),
        "worst_excess": float(excess.max()) if n else 0.0,
    }
    if n:
        i = int(np.argmax(excess))
        st["worst"] = {"index": i, "gpu": float(g[i]), "oracle": float(r[i]), "err": float(diff[i])}
    st["ok"] = bool(st["finite"] and (excess <= 0).all() and st["mean_abs"] <= MEAN_ABS)
    return st


def oracle_pools(case: W.Case):
    """Pools (K, V) as the oracle's own kv_append writes them: sentinel everywhere,
    then the setup tokens, then the step's new tokens."""
    kp = W.sentinel_pool(case)
    vp = W.sentinel_pool(case)
    O.kv_append(kp, vp, case.k_setup, case.v_setup, case.block_tables, case.cu_setup_lens,
                case.setup_ctx_lens, case.block_size)
    O.kv_append(kp, vp, case.k_new, case.v_new, case.block_tables, case.cu_new_lens,
                case.ctx_lens, case.block_size)
    return kp, vp


def oracle_decode(case: W.Case, kp, vp, seqs=None) -> np.ndarray:
    r = case.decode_seqs
    bt = case.block_tables[r.start:r.stop]
    ctx = case.ctx_lens[r.start:r.stop]
    return O.decode(case.q_decode, kp, vp, bt, ctx, case.block_size, case.num_kv_heads,
                    case.head_dim, case.scale, seqs=seqs)


def oracle_prefill(case: W.Case, kp, vp, causal: bool = True) -> np.ndarray:
    r = case.prefill_seqs
    bt = case.block_tables[r.start:r.stop]
    ctx = case.ctx_lens[r.start:r.stop]
    return O.prefill(case.q_prefill, kp, vp, bt, case.cu_q_lens_prefill, ctx, case.block_size,
                     case.num_kv_heads, case.head_dim, case.scale, causal=causal)


def bf16_bits_to_float_py(b: int) -> float:
    """Widen one bf16 pattern with struct (independent of the oracle's numpy widening)."""
    return struct.unpack(">f", struct.pack(">I", (int(b) & 0xFFFF) << 16))[0]


def brute_force_rows(q_rows, k_log, v_log, n_visible, scale):
    """Dense softmax attention by definition, pure Python, over contiguous (never paged)
    K/V: K/V heads are replicated to one per query head, an explicit -inf mask hides
    keys a row may not see, and softmax is exp(x_t) / sum_u exp(x_u).

    q_rows: bits [R, Hq, d]; k_log, v_log: bits [T, Hkv, d]; returns list [R][Hq][d]."""
    r_rows, hq, d = q_rows.shape
    t_keys, hkv, _ = k_log.shape
    group = hq // hkv
    import math

    kf = [[[bf16_bits_to_float_py(k_log[t, g, i]) for i in range(d)] for g in range(hkv)]
          for t in range(t_keys)]
    vf = [[[bf16_bits_to_float_py(v_log[t, g, i]) for i in range(d)] for g in range(hkv)]
          for t in range(t_keys)]
    # replicate each KV head for the query heads of its group
    k_rep = [[kf[t][h // group] for h in range(hq)] for t in range(t_keys)]
    v_rep = [[vf[t][h // group] for h in range(hq)] for t in range(t_keys)]
    out = []
    for r in range(r_rows):
        mask = [0.0 if t < n_visible[r] else -math.inf for t in range(t_keys)]
        row = []
        for h in range(hq):
            qv = [bf16_bits_to_float_py(q_rows[r, h, i]) for i in range(d)]
            x = [scale * sum(qv[i] * k_rep[t][h][i] for i in range(d)) + mask[t]
                 for t in range(t_keys)]
            e = [math.exp(xt) if xt != -math.inf else 0.0 for xt in x]
            den = sum(e)
            if den == 0.0:
                row.append([0.0] * d)
                continue
            row.append([sum(e[t] / den * v_rep[t][h][i] for t in range(t_keys)) for i in range(d)])
        out.append(row)
    return out

"""Parity of pa_rope_kv_append (RoPE of Q and K fused with the K/V append) against the
CPU oracle, on the GPU (marked ``gpu``).

Tolerance, from the arithmetic.  The oracle rotates in fp64 and rounds once to bf16.  The
kernel forms the angle in fp64 but rotates in fp32: cos and sin rounded to fp32, one
product and one fused multiply-add, so before its final rounding it is within
3 * 2^-24 * (|a| + |b|) of the exact value, where (a, b) is the input pair.  Where the pair
nearly cancels that is many bf16 units of the small result, so the bound is absolute in
the input scale: every rotated element must lie within half a bf16 ulp of the exact fp64
value plus 4 * 2^-24 * (|a| + |b|), and at most 0.1% of elements may differ from the
oracle's bf16 at all.  V and every pool byte outside the new slots (sentinels, earlier
tokens) must match bit for bit."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import bf16_dev, bits_host, geometry, i32_dev, sentinel_pools

pytestmark = pytest.mark.gpu

D = 64
THETA = 500000.0


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _assert_rotated_close(got_bits, x_bits, pos, freqs, want_bits, what):
    """Rotated rows ``got_bits`` [T, H, d] of inputs ``x_bits`` at positions ``pos``
    against the exact fp64 rotation (bound above) and the oracle's bf16 ``want_bits``."""
    x = O.bf16_to_f64(x_bits)
    exact = O.rotate(x, pos[:, None], freqs)
    h = D // 2
    scale = np.abs(x[..., :h]) + np.abs(x[..., h:])
    scale = np.concatenate([scale, scale], axis=-1)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 2.0 ** -126))) - 7)
    bound = 0.5 * ulp + 4 * 2.0 ** -24 * scale
    err = np.abs(O.bf16_to_f64(got_bits) - exact)
    worst = np.max(err / bound)
    assert worst <= 1.0, f"{what}: error {worst:.3f} x the bound"
    frac = np.count_nonzero(got_bits != want_bits) / got_bits.size
    assert frac <= 1e-3, f"{what}: {frac:.2e} of elements differ from the oracle's bf16"


def _new_slot_mask(case, block_tables):
    """Pool elements (K layout) written by the new rows."""
    mk, mv = np.zeros_like(W.sentinel_pool(case)), np.zeros_like(W.sentinel_pool(case))
    ones = np.full(case.k_new.shape, 0x3F80, np.uint16)
    O.kv_append(mk, mv, ones, ones, block_tables, case.cu_new_lens, case.ctx_lens,
                case.block_size)
    return mk != 0


def _pool_rows(pool, case, block_tables, rows):
    """K rows of the new tokens ``rows`` read back from a pool through the oracle's layout."""
    hkv, bs = case.num_kv_heads, case.block_size
    pos = O.positions(case.cu_new_lens, case.ctx_lens)
    seq = np.searchsorted(case.cu_new_lens, np.arange(case.k_new.shape[0]), side="right") - 1
    offs = np.array([[[O.k_offset(g, sl, i, bs, D) for i in range(D)] for g in range(hkv)]
                     for sl in range(bs)])  # [bs][Hkv][d]
    rows = np.asarray(rows)
    pages = block_tables[seq[rows], pos[rows] // bs]
    return pool[pages[:, None, None], offs[pos[rows] % bs]]


def _q_bits(case, seed):
    t = case.k_new.shape[0]
    return W.normal_bf16([77, seed], t * case.num_q_heads * D).reshape(t, case.num_q_heads, D)


def _oracle(case, q, freqs, block_tables=None):
    kp, vp = W.sentinel_pool(case), W.sentinel_pool(case)
    O.kv_append(kp, vp, case.k_setup, case.v_setup, case.block_tables, case.cu_setup_lens,
                case.setup_ctx_lens, case.block_size)
    bt = case.block_tables if block_tables is None else block_tables
    q_out = O.rope_kv_append(q, case.k_new, case.v_new, kp, vp, bt, case.cu_new_lens,
                             case.ctx_lens, case.block_size, freqs)
    return kp, vp, q_out


def _run(case, q, inv_freq=None, in_place=False, block_tables=None, with_q=True):
    import torch

    import paged_kv_attention_31_amd as pa

    g = geometry(case)
    kp, vp = sentinel_pools(case)
    bt_host = case.block_tables if block_tables is None else block_tables
    bt = i32_dev(bt_host)
    if case.k_setup.shape[0]:
        pa.kv_append(g, bf16_dev(case.k_setup), bf16_dev(case.v_setup), kp, vp,
                     i32_dev(case.block_tables), i32_dev(case.cu_setup_lens),
                     i32_dev(case.setup_ctx_lens))
    qd = bf16_dev(q) if with_q else None
    qo = (qd if in_place else torch.empty_like(qd)) if with_q else None
    fr = None if inv_freq is None else torch.from_numpy(inv_freq).to("cuda:0")
    pa.rope_kv_append(g, qd, qo, bf16_dev(case.k_new), bf16_dev(case.v_new), kp, vp, bt,
                      i32_dev(case.cu_new_lens), i32_dev(case.ctx_lens), rope_theta=THETA,
                      inv_freq=fr)
    torch.cuda.synchronize()
    return bits_host(kp), bits_host(vp), (bits_host(qo) if with_q else None)


def _check(case, q, freqs, **kw):
    kp, vp, qo = _run(case, q, **kw)
    okp, ovp, oqo = _oracle(case, q if kw.get("with_q", True) else None, freqs)
    bt = case.block_tables
    assert np.array_equal(vp, ovp), "V pool differs"
    mask = _new_slot_mask(case, bt)
    assert np.array_equal(kp[~mask], okp[~mask]), "K pool differs outside the new slots"
    pos = O.positions(case.cu_new_lens, case.ctx_lens)
    rows = np.arange(case.k_new.shape[0])
    _assert_rotated_close(_pool_rows(kp, case, bt, rows), case.k_new, pos, freqs,
                          _pool_rows(okp, case, bt, rows), "K rows in the pool")
    if qo is not None:
        _assert_rotated_close(qo, q, pos, freqs, oqo, "rotated Q")


def test_rope_append_prefill_workload():
    case = W.make_case(3)
    _announce("rope_kv_append workload 3 (4608 tokens, positions 0..1023)")
    _check(case, _q_bits(case, 3), O.rope_freqs(D, THETA))


@pytest.mark.parametrize("bs", [16, 32])
def test_rope_append_far_positions(bs):
    # decode-like rows at positions up to 32767 after a setup append, plus a short prompt
    case = W.custom_case([32768, 8192, 700, 3], [2, 1, 64, 3], block_size=bs, kind="prefill",
                         seed=60 + bs)
    _announce(f"rope_kv_append far positions bs={bs}")
    _check(case, _q_bits(case, bs), O.rope_freqs(D, THETA))


def test_rope_append_in_place_and_k_only():
    case = W.custom_case([40, 5, 129], [40, 5, 17], block_size=16, kind="prefill", seed=71)
    q = _q_bits(case, 71)
    _announce("rope_kv_append in place / K only")
    _check(case, q, O.rope_freqs(D, THETA), in_place=True)
    _check(case, q, O.rope_freqs(D, THETA), with_q=False)


def test_rope_append_frequency_table():
    # a rescaled table (low frequencies divided by 8, a smooth band between)
    f = O.rope_freqs(D, THETA)
    wl = 2 * np.pi / f
    s = np.clip((8192.0 / wl - 1.0) / 3.0, 0.0, 1.0)
    table = ((1 - s) * f / 8.0 + s * f).astype(np.float32)
    case = W.custom_case([3000, 64], [3000, 64], block_size=32, kind="prefill", seed=72)
    _announce("rope_kv_append with a frequency table")
    _check(case, _q_bits(case, 72), table.astype(np.float64), inv_freq=table)


def test_rope_append_out_of_range_page_is_dropped():
    case = W.custom_case([48, 20], [48, 20], block_size=16, kind="prefill", seed=73)
    bt = case.block_tables.copy()
    bt[0, 1] = case.num_pages + 5  # positions 16..31 of sequence 0 have no valid page
    q = _q_bits(case, 73)
    _announce("rope_kv_append out-of-range page id")
    kp, vp, qo = _run(case, q, block_tables=bt)
    # the oracle: every row but those (the positions without a page), appended one by one
    keep = np.ones(case.k_new.shape[0], bool)
    keep[16:32] = False
    okp, ovp = W.sentinel_pool(case), W.sentinel_pool(case)
    cu, ctx = case.cu_new_lens, case.ctx_lens
    freqs = O.rope_freqs(D, THETA)
    pos = O.positions(cu, ctx)
    k_rot = O.f64_to_bf16(O.rotate(O.bf16_to_f64(case.k_new), pos[:, None], freqs))
    for s in range(2):
        for j in range(cu[s], cu[s + 1]):
            if not keep[j]:
                continue
            O.kv_append(okp, ovp, k_rot[j:j + 1], case.v_new[j:j + 1], bt[s:s + 1],
                        np.array([0, 1]), np.array([pos[j] + 1]), 16)
    assert np.array_equal(vp, ovp)
    rows = np.nonzero(keep)[0]
    mk, mv = np.zeros_like(kp), np.zeros_like(vp)
    for j in rows:
        s = int(np.searchsorted(cu, j, side="right") - 1)
        O.kv_append(mk, mv, np.full((1, case.num_kv_heads, D), 0x3F80, np.uint16),
                    np.full((1, case.num_kv_heads, D), 0x3F80, np.uint16), bt[s:s + 1],
                    np.array([0, 1]), np.array([pos[j] + 1]), 16)
    touched = mk != 0
    assert np.array_equal(kp[~touched], okp[~touched]), "K pool differs outside the kept slots"
    _assert_rotated_close(_pool_rows(kp, case, bt, rows), case.k_new[rows], pos[rows], freqs,
                          _pool_rows(okp, case, bt, rows), "K rows in the pool")
    _assert_rotated_close(qo, q, pos, freqs,
                          O.f64_to_bf16(O.rotate(O.bf16_to_f64(q), pos[:, None], freqs)),
                          "rotated Q (rows without a page too)")

"""Pins for the RoPE oracle (oracle/rope.py): each test checks it against something other
than itself -- a library routine, closed forms, invariants, brute force.  CPU only."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import workloads as W

D = 64


def _rng(seed):
    return np.random.default_rng(seed)


def test_freqs_closed_form():
    for theta in (10000.0, 500000.0):
        f = O.rope_freqs(D, theta)
        assert f.shape == (D // 2,) and f[0] == 1.0
        # constant ratio theta^(2/d) between neighbours, strictly decreasing
        r = f[:-1] / f[1:]
        assert np.allclose(r, theta ** (2.0 / D), rtol=1e-13, atol=0)
        # f_i^(d/2) = theta^(-i): exponent identity
        i = np.arange(D // 2)
        assert np.allclose(np.log(f) * (D / 2), -i * np.log(theta), rtol=1e-12, atol=1e-12)


def test_position_zero_is_identity_bitwise():
    x = W.normal_bf16([7, 0], 5 * 3 * D).reshape(5, 3, D)
    y = O.f64_to_bf16(O.rotate(O.bf16_to_f64(x), np.zeros((5, 1)), O.rope_freqs(D, 500000.0)))
    assert np.array_equal(y, x)


def test_rotation_is_complex_multiplication():
    r = _rng(1)
    x = r.standard_normal((9, 4, D))
    pos = r.integers(0, 40000, size=(9, 1))
    f = O.rope_freqs(D, 500000.0)
    got = O.rotate(x, pos, f)
    z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * pos[..., None] * f)
    want = np.concatenate([z.real, z.imag], axis=-1)
    assert np.max(np.abs(got - want)) < 1e-12


def test_pair_norms_kept_and_relative_position():
    r = _rng(2)
    f = O.rope_freqs(D, 10000.0)
    q, k = r.standard_normal(D), r.standard_normal(D)
    for m, n in ((0, 0), (5, 3), (1000, 17), (31000, 30999)):
        qm, kn = O.rotate(q, np.array(m), f), O.rotate(k, np.array(n), f)
        # pair norms
        h = D // 2
        assert np.allclose(qm[:h] ** 2 + qm[h:] ** 2, q[:h] ** 2 + q[h:] ** 2, rtol=1e-12)
        # <R(m) q, R(n) k> = <R(m - n) q, k>
        assert abs(qm @ kn - O.rotate(q, np.array(m - n), f) @ k) < 1e-9


def _nearest_bf16_brute(x: float) -> int:
    """The bf16 pattern nearest to x (ties to even mantissa) by checking every pattern
    within two steps of x's fp32 truncation."""
    t = np.array([x], np.float64).astype(np.float32)
    base = int(t.view(np.uint32)[0]) >> 16
    best, best_err = None, None
    for c in range(base - 2, base + 3):
        c &= 0xFFFF
        v = float(O.bf16_to_f64(np.array([c], np.uint16))[0])
        if not np.isfinite(v):
            continue
        err = abs(v - x)
        if best is None or err < best_err or (err == best_err and (c & 1) == 0):
            best, best_err = c, err
    return best


def test_f64_to_bf16_against_brute_force():
    r = _rng(3)
    xs = list(r.standard_normal(2000) * 10.0 ** r.integers(-30, 30, 2000))
    # exact bf16 values, exact midpoints (ties), and values a hair off a midpoint
    for b in (0x3F80, 0x3F81, 0x4049, 0xBF7F, 0x0080, 0x7F7E):
        lo = float(O.bf16_to_f64(np.array([b], np.uint16))[0])
        hi = float(O.bf16_to_f64(np.array([b + 1], np.uint16))[0])
        mid = (lo + hi) / 2
        xs += [lo, mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf),
               mid + (hi - lo) * 2.0 ** -30, mid - (hi - lo) * 2.0 ** -30]
    xs = np.array(xs, np.float64)
    got = O.f64_to_bf16(xs)
    want = np.array([_nearest_bf16_brute(v) for v in xs], np.uint16)
    assert np.array_equal(got, want)


def test_positions_follow_the_append_rule():
    cu = np.array([0, 3, 3, 4])
    ctx = np.array([10, 5, 1])
    assert O.positions(cu, ctx).tolist() == [7, 8, 9, 0]


@pytest.mark.parametrize("bs", [16, 32])
def test_fused_append_equals_plain_append_of_rotated_rows(bs):
    case = W.custom_case([5, 40, 1], [5, 9, 1], block_size=bs, kind="prefill", seed=11)
    f = O.rope_freqs(D, 500000.0)
    kp1, vp1 = W.sentinel_pool(case), W.sentinel_pool(case)
    kp2, vp2 = W.sentinel_pool(case), W.sentinel_pool(case)
    q = W.normal_bf16([99, 1], case.k_new.shape[0] * case.num_q_heads * D).reshape(
        case.k_new.shape[0], case.num_q_heads, D)
    q_out = O.rope_kv_append(q, case.k_new, case.v_new, kp1, vp1, case.block_tables,
                             case.cu_new_lens, case.ctx_lens, bs, f)
    # the same thing composed from independent pieces: rotate via complex numbers
    pos = np.concatenate([np.arange(c - n, c) for c, n in zip(case.ctx_lens,
                                                              np.diff(case.cu_new_lens))])
    def rot(bits):
        x = O.bf16_to_f64(bits)
        z = (x[..., : D // 2] + 1j * x[..., D // 2:]) * np.exp(1j * pos[:, None, None] * f)
        return O.f64_to_bf16(np.concatenate([z.real, z.imag], axis=-1))
    O.kv_append(kp2, vp2, rot(case.k_new), case.v_new, case.block_tables, case.cu_new_lens,
                case.ctx_lens, bs)
    assert np.array_equal(vp1, vp2)
    # complex vs real rotation may round differently only at fp64 noise next to a tie
    diff = np.abs(kp1.astype(np.int32) - kp2.astype(np.int32))
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 2
    qd = np.abs(q_out.astype(np.int32) - rot(q).astype(np.int32))
    assert qd.max() <= 1 and np.count_nonzero(qd) <= 2

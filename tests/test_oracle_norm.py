"""Pins for the residual + RMSNorm and SiLU-product oracle (oracle/norm.py): closed forms,
invariants and a library routine.  CPU only."""

from __future__ import annotations

import numpy as np
from scipy.special import expit

import oracle as O
import workloads as W


def _bits(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_constant_row_normalises_to_gamma():
    gamma = W.normal_bf16([60, 0], 64)
    for c in (3.0, -0.5, 1e-3):
        x = _bits(np.full((2, 64), c))
        out, h = O.residual_rmsnorm(x, None, gamma, 0.0)
        want = O.f64_to_bf16(np.sign(c) * O.bf16_to_f64(gamma))
        assert np.array_equal(out, np.stack([want, want]))
        assert np.array_equal(h, x)


def test_scale_invariance_and_unit_rms():
    x = W.normal_bf16([60, 1], 4 * 256).reshape(4, 256)
    ones = _bits(np.ones(256))
    out, _ = O.residual_rmsnorm(x, None, ones, 0.0)
    # scaling by a power of two is exact in bf16 and leaves the result unchanged
    out2, _ = O.residual_rmsnorm(_bits(O.bf16_to_f64(x) * 8.0), None, ones, 0.0)
    assert np.array_equal(out, out2)
    # before rounding the row has RMS 1: after rounding within bf16 precision
    y = O.bf16_to_f64(out)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, atol=4e-3)


def test_residual_is_added_then_rounded():
    x = W.normal_bf16([60, 2], 3 * 128).reshape(3, 128)
    r = W.normal_bf16([60, 3], 3 * 128).reshape(3, 128)
    gamma = W.normal_bf16([60, 4], 128)
    out, h = O.residual_rmsnorm(x, r, gamma, 1e-5)
    # the two steps apart: the rounded sum (two bf16 values add exactly in fp64), then the
    # plain normalisation of it
    h2 = O.f64_to_bf16(O.bf16_to_f64(x) + O.bf16_to_f64(r))
    assert np.array_equal(h, h2)
    out2, _ = O.residual_rmsnorm(h2, None, gamma, 1e-5)
    assert np.array_equal(out, out2)
    # and eps enters once: a larger eps shrinks every row
    small, _ = O.residual_rmsnorm(h2, None, _bits(np.ones(128)), 1e-5)
    big, _ = O.residual_rmsnorm(h2, None, _bits(np.ones(128)), 10.0)
    assert np.all(np.abs(O.bf16_to_f64(big)) <= np.abs(O.bf16_to_f64(small)))


def test_silu_against_the_logistic_function():
    g = W.normal_bf16([60, 5], 4096)
    u = W.normal_bf16([60, 6], 4096)
    gf, uf = O.bf16_to_f64(g), O.bf16_to_f64(u)
    want = O.f64_to_bf16(gf * expit(gf) * uf)
    assert np.array_equal(O.silu_mul(g, u), want)


def test_silu_special_values():
    one = _bits([1.0])
    for z, expect in ((0.0, 0.0), (40.0, 40.0), (-40.0, 0.0)):
        got = O.bf16_to_f64(O.silu_mul(_bits([z]), one))[0]
        assert abs(got - expect) <= 1e-12 + abs(expect) * 2.0 ** -8

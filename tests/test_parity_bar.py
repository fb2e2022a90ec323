"""The parity bar itself (CPU): max-abs 1e-2 and mean-abs 1e-3 over all elements, with
elements at |oracle| >= 4 -- where two neighbouring bf16 values lie 2^-5 apart, so even a
correctly rounded output can miss by 2^-6 -- held to half a bf16 unit (+1e-3) and
counted rather than passed silently."""

from __future__ import annotations

import numpy as np

from tests.helpers import MAX_ABS, MEAN_ABS, bf16_half_unit, parity_stats


def test_half_unit_follows_the_bf16_format():
    # 8 significant bits: spacing 2^(e-7) on [2^e, 2^(e+1)), half of it 2^(e-8)
    x = np.array([1.0, 1.99, 2.0, 3.5, 4.0, 7.9, 0.5, -3.0, 1e-3])
    e = np.floor(np.log2(np.abs(x)))
    assert np.array_equal(bf16_half_unit(x), 2.0 ** (e - 8))
    assert bf16_half_unit(np.array([5.0]))[0] == 2.0 ** -6 > MAX_ABS


def test_flat_bar_below_four():
    ref = np.full(1000, 3.0)
    gpu = ref.astype(np.float32).copy()
    gpu[7] += 0.0099
    st = parity_stats(gpu, ref)
    assert st["ok"] and st["n_abs_ge_2"] == 1000 and st["n_abs_ge_4"] == 0
    gpu[7] = 3.0 + 0.0101
    st = parity_stats(gpu, ref)
    assert not st["ok"] and st["worst"]["index"] == 7


def test_counted_exceptions_at_four_and_above():
    ref = np.concatenate([np.full(999, 0.1), [5.0]])
    gpu = ref.astype(np.float32).copy()
    gpu[-1] = np.float32(5.0 + 0.0150)  # beyond 1e-2, within half a unit (2^-6) + 1e-3
    st = parity_stats(gpu, ref)
    assert st["ok"] and st["n_abs_ge_4"] == 1 and st["n_r13_over_max_abs"] == 1
    assert st["max_abs"] > MAX_ABS and st["max_abs_below_r13"] == 0.0
    gpu[-1] = np.float32(5.0 + 0.018)  # more than half a unit off: a real error
    assert not parity_stats(gpu, ref)["ok"]


def test_mean_bar_and_non_finite():
    ref = np.zeros(100)
    gpu = np.full(100, 1.1e-3, np.float32)
    st = parity_stats(gpu, ref)
    assert st["max_abs"] < MAX_ABS and st["mean_abs"] > MEAN_ABS and not st["ok"]
    gpu = np.zeros(100, np.float32)
    gpu[3] = np.nan
    assert not parity_stats(gpu, ref)["ok"]

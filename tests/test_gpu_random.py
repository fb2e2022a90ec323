"""Seeded random batches (marked ``gpu``): per case, the block size, head counts, number of
sequences, their lengths, decode or prefill, the decode partition, prefill causality and
key pieces are drawn from a fixed seed.  The pools after the appends must equal the
oracle's bit for bit, and every output row must meet the parity bar against the oracle.
Decode batches without empty contexts also run pa_decode_append, which must give the same
outputs and pools bit for bit.  The draws cover combinations the hand-picked cases do not
(other head counts with key pieces, empty contexts beside long ones, one-token chunks behind
long prefixes)."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import GpuCase, assert_close, bits_host
from tests.helpers import oracle_decode, oracle_pools, oracle_prefill
from tests.test_gpu_decode_append import _both_paths

pytestmark = pytest.mark.gpu

N_CASES = 40


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _draw(i: int) -> dict:
    rng = np.random.default_rng([150, i])
    heads = [(32, 8), (32, 8), (8, 2), (4, 1), (64, 16)][int(rng.integers(5))]
    d = {"bs": int(rng.choice([16, 32])), "hq": heads[0], "hkv": heads[1]}
    if rng.random() < 0.5:
        n = int(rng.integers(1, 25))
        ctx = rng.integers(0, 2500, n)
        ctx[rng.random(n) < 0.1] = 0  # empty contexts beside the others
        d.update(kind="decode", ctx=ctx.tolist(), new=[1 if c > 0 else 0 for c in ctx],
                 part=int(rng.choice([0, 0, 64, 128, 256, 1024])))
    else:
        n = int(rng.integers(1, 7))
        ctx = rng.integers(1, 1500, n)
        new = [int(rng.integers(1, min(int(c), 200) + 1)) for c in ctx]
        d.update(kind="prefill", ctx=ctx.tolist(), new=new, causal=bool(rng.random() < 0.75),
                 splits=int(rng.choice([0, 0, 1, 2, 3, 8])))
    return d


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_batch(i):
    d = _draw(i)
    _announce(f"random case {i}: {d}")
    case = W.custom_case(d["ctx"], d["new"], kind=d["kind"], block_size=d["bs"],
                         num_q_heads=d["hq"], num_kv_heads=d["hkv"], seed=200 + i)
    g = GpuCase(case)
    kp, vp = oracle_pools(case)
    assert np.array_equal(bits_host(g.kp), kp) and np.array_equal(bits_host(g.vp), vp)
    if d["kind"] == "decode":
        out = g.decode(partition_tokens=d["part"])
        ref = oracle_decode(case, kp, vp)
        if min(d["ctx"]) > 0:  # one new token per sequence: the fused call must match
            a, b, same, _, _ = _both_paths(case, d["part"])
            assert np.array_equal(a, b) and same, "pa_decode_append differs"
            assert np.array_equal(a, bits_host(out))
    else:
        out = g.prefill(causal=d["causal"], kv_splits=d["splits"])
        ref = oracle_prefill(case, kp, vp, causal=d["causal"])
    mx, mean = assert_close(out, ref, f"random case {i}")
    _announce(f"random case {i}: max-abs {mx:.2e} mean-abs {mean:.2e}")

"""Parity of pa_residual_rmsnorm and pa_silu_mul against the CPU oracle (marked ``gpu``).

Tolerance, from the arithmetic: the kernels work in fp32 and round once to bf16; the sum
of squares over H terms is off by at most H * 2^-24 relative (6e-5 at H = 2048, far less
in practice), exp and the division by a few fp32 ulps.  So every element must lie within
one bf16 unit of the oracle (fp64, one rounding), and at most 1% of them (RMSNorm) or
0.1% (residual sum, SiLU product) may differ from it at all."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import bf16_dev, bits_host

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _key(bits):
    b = bits.astype(np.int64)
    return np.where(b >= 0x8000, -(b - 0x8000), b)


def _within_one_ulp(got, want, frac, what):
    d = np.abs(_key(got) - _key(want))
    assert d.max(initial=0) <= 1, f"{what}: {int(d.max())} units off"
    f = np.count_nonzero(d) / max(d.size, 1)
    assert f <= frac, f"{what}: {f:.2e} of elements differ"


# (4622, 2048): the 1B shape; the others reach every register budget of the kernel (rows
# of up to 4, 8 and 16 chunks per lane), ragged chunk counts and row counts that leave a
# workgroup part empty.  Above 1024 rows (four row streams per compute unit on 256 compute
# units) a wave takes several rows, two per pass with the second maybe past the end: one to
# nine rows a wave, odd and even counts, full and ragged rows, with and without prefetch.
@pytest.mark.parametrize("rows,hidden", [(4622, 2048), (37, 8), (5, 136), (3, 8192),
                                         (66, 2056), (9, 4096), (130, 6144), (2500, 4096),
                                         (3001, 3000), (2071, 1032), (9000, 2048),
                                         (1100, 8192)])
@pytest.mark.parametrize("with_res", [True, False])
def test_residual_rmsnorm(rows, hidden, with_res):
    import torch

    import paged_kv_attention_31_amd as pa

    _announce(f"residual_rmsnorm {rows}x{hidden} residual={with_res}")
    x = W.normal_bf16([70, rows, hidden, 0], rows * hidden).reshape(rows, hidden)
    r = W.normal_bf16([70, rows, hidden, 1], rows * hidden, 2.0).reshape(rows, hidden)
    gm = W.normal_bf16([70, rows, hidden, 2], hidden)
    xd, gd = bf16_dev(x), bf16_dev(gm)
    out = torch.empty_like(xd)
    rd = bf16_dev(r) if with_res else None
    pa.residual_rmsnorm(xd, gd, out, residual_in=rd, residual_out=rd, eps=1e-5)  # in place
    torch.cuda.synchronize()
    want, h = O.residual_rmsnorm(x, r if with_res else None, gm, 1e-5)
    if with_res:
        _within_one_ulp(bits_host(rd), h, 1e-3, "residual sum")
    _within_one_ulp(bits_host(out), want, 1e-2, "normalised rows")


# enough rows for four chunks per thread (4622 x 8192, 600 x 8200 with a ragged last column
# group) and too few (7 x 1000, 2 x 20000 over several column groups, 1 x 8)
@pytest.mark.parametrize("rows,width,fused", [(4622, 8192, False), (4622, 8192, True),
                                              (600, 8200, True), (7, 1000, False),
                                              (2, 20000, True), (1, 8, True)])
def test_silu_mul(rows, width, fused):
    import torch

    import paged_kv_attention_31_amd as pa

    _announce(f"silu_mul {rows}x{width} fused={fused}")
    g = W.normal_bf16([71, rows, width, 0], rows * width, 3.0).reshape(rows, width)
    u = W.normal_bf16([71, rows, width, 1], rows * width).reshape(rows, width)
    if fused:  # one [rows, 2 width] gate|up buffer
        gu = bf16_dev(np.concatenate([g, u], axis=1))
        gd, ud = gu[:, :width], gu[:, width:]
    else:
        gd, ud = bf16_dev(g), bf16_dev(u)
    out = torch.empty((rows, width), dtype=torch.bfloat16, device="cuda:0")
    pa.silu_mul(gd, ud, out)
    torch.cuda.synchronize()
    _within_one_ulp(bits_host(out), O.silu_mul(g, u), 1e-3, "silu(g) * u")


def test_silu_mul_strided_out():
    """The product written into the left half of a wider buffer; the right half untouched."""
    import torch

    import paged_kv_attention_31_amd as pa

    rows, width = 513, 3072
    _announce(f"silu_mul {rows}x{width} into a [{rows}, {2 * width}] buffer")
    g = W.normal_bf16([71, rows, width, 2], rows * width, 3.0).reshape(rows, width)
    u = W.normal_bf16([71, rows, width, 3], rows * width).reshape(rows, width)
    wide = torch.full((rows, 2 * width), 7.0, dtype=torch.bfloat16, device="cuda:0")
    pa.silu_mul(bf16_dev(g), bf16_dev(u), wide[:, :width])
    torch.cuda.synchronize()
    host = bits_host(wide)
    _within_one_ulp(host[:, :width], O.silu_mul(g, u), 1e-3, "silu(g) * u")
    assert np.all(host[:, width:] == W.f32_to_bf16_bits(np.float32([7.0]))[0])

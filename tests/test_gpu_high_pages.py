"""Pools past 4 GiB (marked ``gpu``): the same batches with every page id moved up far
enough that the used pages sit more than 5 GiB into each pool must give, bit for bit, the
outputs and page contents of the batches at the bottom of the pools, through pa_kv_append,
pa_decode, pa_prefill, pa_rope_kv_append, pa_decode_append and pa_copy_pages.  A page's
content and the order of every computation do not depend on its id, so any difference is a
page address formed in 32 bits somewhere."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import GpuCase, bf16_dev, bits_host, geometry, i32_dev, sentinel_pools

pytestmark = pytest.mark.gpu

LIFT_BYTES = 5 << 30  # the used pages start this far into each pool


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


def _lift_pages(case: W.Case) -> int:
    return LIFT_BYTES // (case.block_size * case.num_kv_heads * case.head_dim * 2)


def _lifted(case: W.Case, off: int) -> W.Case:
    return dataclasses.replace(case, num_pages=case.num_pages + off,
                               block_tables=(case.block_tables + off).astype(np.int32),
                               sentinel_page=case.sentinel_page + off)


def _same(a, b) -> bool:
    import torch

    return bool(torch.equal(a.view(torch.int16), b.view(torch.int16)))


def _free():
    import torch

    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_append_and_attention_past_4gib(bs, kind):
    if kind == "decode":
        case = W.custom_case([3000, 517, 1, 2048, 64], [1] * 5, block_size=bs, seed=120 + bs)
    else:
        case = W.custom_case([1500, 700], [300, 700], kind="prefill", block_size=bs,
                             seed=122 + bs)
    off = _lift_pages(case)
    _announce(f"{kind} bs={bs}: page ids lifted by {off} ({LIFT_BYTES >> 30} GiB)")
    lo = GpuCase(case)
    out_lo = lo.decode() if kind == "decode" else lo.prefill()
    hi = GpuCase(_lifted(case, off))
    out_hi = hi.decode() if kind == "decode" else hi.prefill()
    import torch

    torch.cuda.synchronize()
    assert np.array_equal(bits_host(out_lo), bits_host(out_hi))
    assert _same(hi.kp[off:], lo.kp) and _same(hi.vp[off:], lo.vp)
    del lo, hi, out_lo, out_hi
    _free()


def test_decode_append_and_copy_past_4gib():
    import torch

    import paged_kv_attention_31_amd as pa

    case = W.custom_case([1000, 33, 2048, 1], [1] * 4, block_size=32, seed=126)
    off = _lift_pages(case)
    n, hkv, d = case.n_seqs, case.num_kv_heads, case.head_dim
    _announce(f"decode_append + copy_pages bs=32: page ids lifted by {off}")

    def run(c: W.Case):
        geom = geometry(c)
        kp, vp = sentinel_pools(c)
        bt, ctx = i32_dev(c.block_tables), i32_dev(c.ctx_lens)
        pa.kv_append(geom, bf16_dev(c.k_setup), bf16_dev(c.v_setup), kp, vp, bt,
                     i32_dev(c.cu_setup_lens), i32_dev(c.setup_ctx_lens))
        out = torch.empty((n, c.num_q_heads, d), dtype=torch.bfloat16, device="cuda:0")
        pa.decode_append(geom, out, bf16_dev(c.q_decode), bf16_dev(c.k_new.reshape(n, hkv, d)),
                         bf16_dev(c.v_new.reshape(n, hkv, d)), kp, vp, bt, ctx,
                         int(c.ctx_lens.max()), c.scale)
        return geom, kp, vp, out

    _, kp_lo, vp_lo, out_lo = run(case)
    geom, kp_hi, vp_hi, out_hi = run(_lifted(case, off))
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(out_lo), bits_host(out_hi))
    assert _same(kp_hi[off:], kp_lo) and _same(vp_hi[off:], vp_lo)
    # copy the first pages of sequence 2 to the five free pages just below the lifted ones
    # (still past 4 GiB)
    src = case.block_tables[2, :5].astype(np.int32) + off
    dst = np.arange(off - 5, off, dtype=np.int32)
    pa.copy_pages(geom, kp_hi, vp_hi, i32_dev(src), i32_dev(dst))
    torch.cuda.synchronize()
    for s_, d_ in zip(src.tolist(), dst.tolist()):
        assert _same(kp_hi[d_], kp_hi[s_]) and _same(vp_hi[d_], vp_hi[s_])
    del kp_lo, vp_lo, kp_hi, vp_hi, out_lo, out_hi
    _free()


@pytest.mark.parametrize("bs", [16, 32])
def test_rope_append_past_4gib(bs):
    import torch

    import paged_kv_attention_31_amd as pa

    case = W.custom_case([700, 129, 1024], [700, 1, 300], kind="prefill", block_size=bs,
                         seed=128 + bs)
    off = _lift_pages(case)
    hq, hkv, d = case.num_q_heads, case.num_kv_heads, case.head_dim
    t = int(case.cu_new_lens[-1])
    _announce(f"rope_kv_append bs={bs}: page ids lifted by {off}")
    q = bf16_dev(W.normal_bf16([77, 128 + bs], t * hq * d).reshape(t, hq, d))

    def run(c: W.Case):
        geom = geometry(c)
        kp, vp = sentinel_pools(c)
        q_out = torch.empty_like(q)
        pa.rope_kv_append(geom, q, q_out, bf16_dev(c.k_new.reshape(t, hkv, d)),
                          bf16_dev(c.v_new.reshape(t, hkv, d)), kp, vp, i32_dev(c.block_tables),
                          i32_dev(c.cu_new_lens), i32_dev(c.ctx_lens))
        return kp, vp, q_out

    kp_lo, vp_lo, q_lo = run(case)
    kp_hi, vp_hi, q_hi = run(_lifted(case, off))
    torch.cuda.synchronize()
    assert _same(q_hi, q_lo)
    assert _same(kp_hi[off:], kp_lo) and _same(vp_hi[off:], vp_lo)
    del kp_lo, vp_lo, kp_hi, vp_hi, q_lo, q_hi, q
    _free()

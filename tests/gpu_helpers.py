"""GPU-side plumbing for the parity tests: upload a generated batch, run the library
over it, and compare with the oracle.  Test infrastructure only."""

from __future__ import annotations

import numpy as np

import workloads as W
from tests.helpers import MAX_ABS, MEAN_ABS, parity_stats  # noqa: F401  (the bar)


def torch_mod():
    import torch

    return torch


def dev():
    return torch_mod().device("cuda:0")


def bf16_dev(bits: np.ndarray):
    t = torch_mod()
    a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
    return t.from_numpy(a).to(dev()).view(t.bfloat16)


def i32_dev(a: np.ndarray):
    t = torch_mod()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def bits_host(x) -> np.ndarray:
    """bf16 device tensor -> uint16 numpy bits."""
    t = torch_mod()
    return x.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def f32_host(x) -> np.ndarray:
    return x.float().cpu().numpy()


def geometry(case: W.Case):
    import paged_kv_attention_31_amd as pa

    return pa.Geometry(case.num_pages, case.block_size, case.num_q_heads, case.num_kv_heads,
                       case.head_dim)


def sentinel_pools(case: W.Case):
    t = torch_mod()
    e = W.page_elems(case)
    k = t.full((case.num_pages, e), W.SENTINEL_BITS, dtype=t.int16, device=dev()).view(t.bfloat16)
    v = t.full((case.num_pages, e), W.SENTINEL_BITS, dtype=t.int16, device=dev()).view(t.bfloat16)
    return k, v


class GpuCase:
    """A generated batch on the device, with the library's pools after setup + step
    appends."""

    def __init__(self, case: W.Case, pools=None):
        import paged_kv_attention_31_amd as pa

        self.case = case
        self.geom = geometry(case)
        self.bt = i32_dev(case.block_tables)
        self.ctx = i32_dev(case.ctx_lens)
        self.kp, self.vp = pools if pools is not None else sentinel_pools(case)
        hkv, d = case.num_kv_heads, case.head_dim
        if case.k_setup.shape[0]:
            pa.kv_append(self.geom, bf16_dev(case.k_setup), bf16_dev(case.v_setup), self.kp,
                         self.vp, self.bt, i32_dev(case.cu_setup_lens),
                         i32_dev(case.setup_ctx_lens))
        self.k_new = bf16_dev(case.k_new.reshape(-1, hkv, d))
        self.v_new = bf16_dev(case.v_new.reshape(-1, hkv, d))
        self.cu_new = i32_dev(case.cu_new_lens)
        self.append_step()
        r = case.decode_seqs
        self.dec_bt = self.bt[r.start:r.stop]
        self.dec_ctx = self.ctx[r.start:r.stop]
        r = case.prefill_seqs
        self.pre_bt = self.bt[r.start:r.stop]
        self.pre_ctx = self.ctx[r.start:r.stop]
        self.q_dec = bf16_dev(case.q_decode) if len(case.decode_seqs) else None
        self.q_pre = bf16_dev(case.q_prefill) if len(case.prefill_seqs) else None
        self.cu_q = i32_dev(case.cu_q_lens_prefill)

    def append_step(self):
        import paged_kv_attention_31_amd as pa

        if self.case.k_new.shape[0]:
            pa.kv_append(self.geom, self.k_new, self.v_new, self.kp, self.vp, self.bt,
                         self.cu_new, self.ctx)

    def decode(self, partition_tokens: int = 0, max_ctx=None):
        import paged_kv_attention_31_amd as pa

        t = torch_mod()
        c = self.case
        r = c.decode_seqs
        out = t.empty((len(r), c.num_q_heads, c.head_dim), dtype=t.bfloat16, device=dev())
        mc = int(c.ctx_lens[r.start:r.stop].max()) if max_ctx is None else max_ctx
        pa.decode(self.geom, out, self.q_dec, self.kp, self.vp, self.dec_bt, self.dec_ctx, mc,
                  c.scale, partition_tokens=partition_tokens)
        return out

    def prefill(self, causal: bool = True, kv_splits: int = 0):
        import paged_kv_attention_31_amd as pa

        t = torch_mod()
        c = self.case
        ql = c.q_lens_prefill
        out = t.empty((int(ql.sum()), c.num_q_heads, c.head_dim), dtype=t.bfloat16, device=dev())
        r = c.prefill_seqs
        pa.prefill(self.geom, out, self.q_pre, self.kp, self.vp, self.pre_bt, self.cu_q,
                   self.pre_ctx, int(ql.max()), int(c.ctx_lens[r.start:r.stop].max()), c.scale,
                   causal=causal, kv_splits=kv_splits)
        return out


def errors(gpu_out, ref_f64: np.ndarray):
    """(max-abs, mean-abs) of the bf16 GPU output (widened to fp32) against the oracle's
    fp64 result rounded to fp32."""
    st = parity_stats(f32_host(gpu_out), ref_f64)
    return st["max_abs"], st["mean_abs"]


def assert_close(gpu_out, ref_f64: np.ndarray, what: str = ""):
    """The parity bar (``tests.helpers.parity_stats``) over every element; prints the
    element counts at |oracle| >= 2 and >= 4 and how many of the latter exceed 1e-2."""
    st = parity_stats(f32_host(gpu_out), ref_f64)
    msg = (f"{what}: max-abs {st['max_abs']:.3e} (below |o|=4: {st['max_abs_below_r13']:.3e}) "
           f"mean-abs {st['mean_abs']:.3e}; |o|>=2: {st['n_abs_ge_2']}, |o|>=4: "
           f"{st['n_abs_ge_4']} ({st['n_r13_over_max_abs']} beyond 1e-2) of {st['n']}")
    assert st["finite"], f"{what}: non-finite output"
    assert st["ok"], msg + f"; worst {st.get('worst')}"
    if st["n_abs_ge_4"]:
        print(f"[gpu-test] R13 {msg}", flush=True)
    return st["max_abs"], st["mean_abs"]

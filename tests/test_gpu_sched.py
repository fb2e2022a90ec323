"""The slot scheduler driving the kernels (marked ``gpu``): every step's plan from
pa_sched_step goes, as is, to pa_kv_append and then pa_prefill or pa_decode; every output
row must match the oracle's attention over the request's own tokens, taken contiguously
from the generator (not from the pages), so a wrong block table, position or context
length in a plan shows up as a wrong row.  One run serves its decode steps with
pa_decode_append (append and attention in one launch).  One run appends through pa_rope_kv_append
instead: then Q and every cached K are turned by their positions (oracle: the rotation in
fp64, rounded once to bf16), so the plans' positions are checked as well.

Tolerance: the parity bar, element by element over the whole run (max-abs 1e-2, mean-abs
1e-3; elements with |oracle| >= 4, where half a bf16 unit exceeds 1e-2, are held to half a
bf16 unit and counted).  The first rows of every prompt (prompts start at 1 token) see a
handful of keys, the case in which the kernels' two-term probabilities matter."""

from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests.gpu_helpers import bf16_dev, f32_host, i32_dev
from tests.helpers import parity_stats

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 64
SCALE = 0.125


def _announce(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.mark.parametrize("bs,slots,chunk,rope,fused", [(16, 4, 96, False, False),
                                                        (32, 6, 200, False, True),
                                                        (16, 5, 128, True, False)])
def test_scheduler_plans_drive_the_kernels(bs, slots, chunk, rope, fused):
    import torch

    import paged_kv_attention_31_amd as pa

    _announce(f"scheduler-driven run bs={bs} slots={slots} chunk={chunk} rope={rope} "
              f"fused={fused}")
    rng = np.random.default_rng([92, bs])
    n_req, max_blocks, num_pages = 12, 24, 90
    reqs = {}
    for rid in range(n_req):
        p, m = int(rng.integers(1, 300)), int(rng.integers(1, 10))
        L = p + m - 1
        reqs[rid] = dict(
            prompt=p, max_new=m,
            q=W.normal_bf16([92, bs, rid, 0], L * HQ * D).reshape(L, HQ, D),
            k=W.normal_bf16([92, bs, rid, 1], L * HKV * D).reshape(L, HKV, D),
            v=W.normal_bf16([92, bs, rid, 2], L * HKV * D).reshape(L, HKV, D))
        if rope:  # what the kernel attends with: rows turned by position, in bf16
            f = O.rope_freqs(D, 500000.0)
            pos = np.arange(L)
            for name in ("q", "k"):
                r = reqs[rid]
                r[name + "_att"] = O.f64_to_bf16(O.rotate(O.bf16_to_f64(r[name]),
                                                          pos[:, None], f))
        else:
            reqs[rid]["q_att"], reqs[rid]["k_att"] = reqs[rid]["q"], reqs[rid]["k"]
    geom = pa.Geometry(num_pages, bs, HQ, HKV, D)
    e = bs * HKV * D
    kp = torch.full((num_pages, e), W.SENTINEL_BITS, dtype=torch.int16, device="cuda:0").view(
        torch.bfloat16)
    vp = torch.full_like(kp, float("nan"))
    pool = pa.PagePool(num_pages)
    sched = pa.Scheduler(pool, slots, bs, max_blocks, chunk)
    for rid, r in reqs.items():
        sched.submit(rid, r["prompt"], r["max_new"])

    produced = {rid: 0 for rid in reqs}
    kinds = []
    gpu_rows, ref_rows = [], []
    for _ in range(1000):
        plan = sched.step()
        kinds.append(plan.kind)
        if plan.kind == pa.STEP_IDLE:
            if sched.pending() == 0:
                break
            continue
        qs, ks, vs, refs = [], [], [], []
        for k, rid in enumerate(plan.req_ids.tolist()):
            r = reqs[rid]
            ctx = int(plan.ctx_lens[k])
            n = int(plan.cu_new_lens[k + 1] - plan.cu_new_lens[k])
            pos = np.arange(ctx - n, ctx)
            ks.append(r["k"][pos])
            vs.append(r["v"][pos])
            qs.append(r["q"][pos])
            refs.append(O.attention(O.bf16_to_f64(r["q_att"][pos]),
                                    O.bf16_to_f64(r["k_att"][:ctx]),
                                    O.bf16_to_f64(r["v"][:ctx]), pos + 1, SCALE))
            if plan.kind == pa.STEP_DECODE or ctx == r["prompt"]:
                produced[rid] += 1
        bt, ctx_d, cu = (i32_dev(plan.block_tables), i32_dev(plan.ctx_lens),
                         i32_dev(plan.cu_new_lens))
        qd = bf16_dev(np.concatenate(qs))
        kd, vd = bf16_dev(np.concatenate(ks)), bf16_dev(np.concatenate(vs))
        out = torch.empty_like(qd)
        if fused and plan.kind == pa.STEP_DECODE:  # append and attend in one launch
            n = len(plan.req_ids)
            pa.decode_append(geom, out, qd, kd.view(n, HKV, D), vd.view(n, HKV, D), kp, vp, bt,
                             ctx_d, max_ctx_len=plan.max_ctx_len, scale=SCALE)
        else:
            if rope:
                pa.rope_kv_append(geom, qd, qd, kd, vd, kp, vp, bt, cu, ctx_d,
                                  rope_theta=500000.0)
            else:
                pa.kv_append(geom, kd, vd, kp, vp, bt, cu, ctx_d)
            if plan.kind == pa.STEP_PREFILL:
                pa.prefill(geom, out, qd, kp, vp, bt, cu, ctx_d, max_q_len=plan.max_new_len,
                           max_ctx_len=plan.max_ctx_len, scale=SCALE, causal=True)
            else:
                pa.decode(geom, out, qd, kp, vp, bt, ctx_d, max_ctx_len=plan.max_ctx_len,
                          scale=SCALE)
        torch.cuda.synchronize()
        gpu_rows.append(f32_host(out))
        ref_rows.append(np.concatenate(refs))
    assert sched.pending() == 0
    assert produced == {rid: r["max_new"] for rid, r in reqs.items()}
    assert pa.STEP_PREFILL in kinds and pa.STEP_DECODE in kinds
    g = np.concatenate([x.reshape(-1) for x in gpu_rows]).astype(np.float32)
    r = np.concatenate([x.reshape(-1) for x in ref_rows])
    st = parity_stats(g, r)
    _announce(f"max-abs {st['max_abs']:.4g} (below |o|=4: {st['max_abs_below_r13']:.4g}), "
              f"mean-abs {st['mean_abs']:.3g}; |o|>=2: {st['n_abs_ge_2']}, |o|>=4: "
              f"{st['n_abs_ge_4']} ({st['n_r13_over_max_abs']} beyond 1e-2) of {st['n']}")
    assert st["finite"]
    assert st["ok"], f"parity: {st}"
    sched.close()
    assert pool.num_free() == num_pages

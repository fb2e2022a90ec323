"""One step of the path (append, chunked prefill, split decode) captured in a HIP graph
and replayed (marked ``gpu``): every replay, with eager work and synchronisations between
replays, must reproduce the eager outputs and pools bit for bit.  Captured once in one
stream and once with the prefill forked onto a second stream, concurrent with the decode,
and joined back."""

from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from tests.gpu_helpers import GpuCase, bits_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("overlap", [False, True])
def test_graph_replays_match_eager(overlap):
    import torch

    import paged_kv_attention_31_amd as pa

    print(f"[gpu-test] graph capture of append + prefill + decode, overlap={overlap}",
          flush=True)
    dec = GpuCase(W.custom_case([1, 700, 3000, 65, 129], [1] * 5, block_size=32, seed=95))
    pre = GpuCase(W.custom_case([600, 97], [200, 97], block_size=32, kind="prefill", seed=96))
    cd, cp = dec.case, pre.case
    n_dec, n_q = len(cd.decode_seqs), int(cp.q_lens_prefill.sum())
    mc_dec, mc_pre = int(cd.ctx_lens.max()), int(cp.ctx_lens.max())
    max_q = int(cp.q_lens_prefill.max())
    part = 128  # several workers per sequence: partials and the merge kernel run
    ws_d = torch.empty(max(pa.decode_workspace_bytes(dec.geom, n_dec, mc_dec, part), 1),
                       dtype=torch.uint8, device="cuda:0")
    ws_p = torch.empty(max(pa.prefill_workspace_bytes(pre.geom, 2, max_q, mc_pre, 4), 1),
                       dtype=torch.uint8, device="cuda:0")
    out_d = torch.empty((n_dec, 32, 64), dtype=torch.bfloat16, device="cuda:0")
    out_p = torch.empty((n_q, 32, 64), dtype=torch.bfloat16, device="cuda:0")

    side = torch.cuda.Stream()

    def step(stream, fork=False):
        pa.kv_append(dec.geom, dec.k_new, dec.v_new, dec.kp, dec.vp, dec.bt, dec.cu_new, dec.ctx,
                     stream=stream)
        pa.kv_append(pre.geom, pre.k_new, pre.v_new, pre.kp, pre.vp, pre.bt, pre.cu_new, pre.ctx,
                     stream=stream)
        if fork:
            side.wait_stream(stream)
        pa.prefill(pre.geom, out_p, pre.q_pre, pre.kp, pre.vp, pre.pre_bt, pre.cu_q, pre.pre_ctx,
                   max_q, mc_pre, cp.scale, kv_splits=4, workspace=ws_p,
                   stream=side if fork else stream)
        pa.decode(dec.geom, out_d, dec.q_dec, dec.kp, dec.vp, dec.dec_bt, dec.dec_ctx, mc_dec,
                  cd.scale, partition_tokens=part, workspace=ws_d, stream=stream)
        if fork:
            stream.wait_stream(side)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [bits_host(x) for x in (out_d, out_p, dec.kp, dec.vp, pre.kp, pre.vp)]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        step(cap, fork=overlap)
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda:0")
    for rep in range(4):
        out_d.zero_()
        out_p.zero_()
        scratch.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [bits_host(x) for x in (out_d, out_p, dec.kp, dec.vp, pre.kp, pre.vp)]
        for name, g, w in zip(("decode out", "prefill out", "dec K", "dec V", "pre K", "pre V"),
                              got, want):
            assert np.array_equal(g, w), f"replay {rep}: {name} differs from eager"

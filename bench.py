"""Benchmark of the paged-attention hot path on one MI355X.

Default workload: the mixed continuous-batch step over 16 layers (per layer: kv_append
of 640 new tokens, a 512-token causal prefill chunk over 512 cached tokens, and decode
of 128 sequences with contexts uniform in [16, 8192], the first 256 tokens of 32 of
them on shared pages; block size 32; 32 query / 8 KV heads, head_dim 64, bf16).  It is
the one workload that runs every step of the path (append, decode partitions, split-K
merge, chunked prefill), so one step = one pass of the whole path.

    python bench.py [--steps K] [--warmup W]
                    [--workload mixed|decode-long|decode-batched|prefill|rope-append|copy-pages|
                                norm-mlp|serve]

Prints one JSON line.  ``value`` = decode KV bytes read per step / wall time per step
(whole step, all kernels), the step captured once in a HIP graph and replayed (the eager
step time is reported beside it).  ``roofline`` reports the dominant kernel (pa_decode, timed
with HIP events on its stream) against HBM peak; ``roofline_prefill`` reports pa_prefill
against dense bf16 MFMA peak.  The same default run then measures the other targets'
own workloads and adds them to the line: ``roofline_prefill_8prompts`` (pa_prefill on the
8-prompt workload), ``roofline_decode_batched`` and ``roofline_decode_long`` (the
64-sequence and 16 x 32k decode steps, one pa_decode_append launch per layer, with pa_decode
beside it).  ``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload
(layer 0) on a process pool over the host's cores, before the GPU is touched.

``--workload rope-append`` times pa_rope_kv_append alone (RoPE of Q and K fused with the
K/V append) on the 4622 new rows of the prefill workload, against HBM peak, with the
plain pa_kv_append of the same rows beside it.  ``--workload copy-pages`` times
pa_copy_pages (the copy half of copy-on-write) on 4096 block-size-32 pages of both pools.
``--workload norm-mlp`` times pa_silu_mul on a concatenated [4622, 2 x 8192] gate|up buffer
(the prefill workload's tokens at the 1B MLP width) with pa_residual_rmsnorm of the
[4622, 2048] hidden rows beside it.  ``--workload serve`` runs the slot scheduler
(pa_sched_step) over 256 requests (prompts U[128, 1024], U[16, 128] new tokens, 64 slots,
16 layers), each plan uploaded and run through pa_kv_append + pa_prefill, or
pa_decode_append for decode steps;
``value`` is the decode KV-read rate over the scheduled decode launches, with the
scheduler's host time per step and the generated tokens per second of the whole loop.

The pure decode workloads (decode-batched, decode-long) run their step as one
pa_decode_append launch per layer (the one-token append fused into the decode); the step
with pa_kv_append + pa_decode is timed beside it (``step_timing``) and ``roofline_decode_only``
gives pa_decode alone.

No timed launch finds its inputs in a cache: the decode-batched and prefill workloads (one
layer each) walk through 6 and 16 independent copies of their layer, and the kernel-level
workloads cycle back-to-back launches through independent buffer sets of at least 1 GiB
in total, four times the last-level cache, so each launch also pays for the write-back of
the outputs before it, as in a layer-by-layer pass.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "decode KV-read GB/s (%HBM peak); prefill TFLOP/s (%MFMA peak), 1B shape"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KV_BYTES_PER_TOKEN = 2 * 8 * 64 * 2  # K and V, 8 KV heads x 64 dims x bf16, per layer
FLOP_PER_PAIR = 4 * 64 * 32  # QK^T and PV over 32 query heads, per visible (query, key)

WORKLOADS = {
    "mixed": 5,
    "decode-long": 4,
    "decode-batched": 2,
    "prefill": 3,
    "rope-append": 3,
    "copy-pages": 0,
    "norm-mlp": 0,
    "serve": 0,
}
NORM_ROWS, HIDDEN, MLP_WIDTH = 4622, 2048, 8192
# Independent copies of a one-layer workload that a step walks through, so that its
# working set (pools, q, outputs) exceeds the 256 MB last-level cache and every layer's
# bytes come from HBM, as they do in the 16-layer mixed step.
LAYER_COPIES = {2: 6, 3: 16}
# Kernel-level workloads rotate over independent copies of their buffers totalling at least
# this many bytes, so that back-to-back launches find nothing in the L2s or the 256 MB
# last-level cache and pay for the write-back of the launches before them, as a layer does.
ROTATE_BYTES = 1 << 30
COPY_PAGES, COPY_BS = 4096, 32
# scheduler-driven serving run: requests with prompts U[128, 1024] (the prefill workload's
# range) and U[16, 128] new tokens through 64 slots, 16 layers, block size 16
SERVE_REQS, SERVE_SLOTS, SERVE_CHUNK, SERVE_BS, SERVE_LAYERS = 256, 64, 2048, 16, 16


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def hbm_traffic(key: str):
    """HBM bytes per launch that rocprofv3 FETCH_SIZE / WRITE_SIZE counters measured for this
    workload's kernel (profiles/hbm_traffic.json, scaled by the 1 GiB copy calibration), or
    None when there is no entry or the kernel source has changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            entry = json.load(f)["entries"][key]
        with open(os.path.join(ROOT, entry["source"]), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, KeyError, ValueError):
        return None
    if digest != entry["source_sha256"]:
        return None
    return round(float(entry["bytes_per_launch"]))


def unique_kv_bytes(case: W.Case) -> int:
    """Decode KV bytes with pages shared by several sequences counted once (the logical
    figure, ``kv_tokens() * 2048``, counts them once per sequence that reads them)."""
    r = case.decode_seqs
    n_shared = len([s for s in case.shared_seqs if r.start <= s < r.stop])
    dup = max(n_shared - 1, 0) * case.shared_prefix_tokens
    return (case.kv_tokens() - dup) * KV_BYTES_PER_TOKEN


def prefill_min_bytes(case: W.Case) -> int:
    """HBM bytes a prefill launch cannot avoid: its q rows read and output rows written once
    (32 heads x 64 dims x bf16 each) and every prefill sequence's K/V read once."""
    p = case.prefill_seqs
    rows = int(case.q_lens_prefill.sum())
    ctx = int(case.ctx_lens[p.start:p.stop].astype(np.int64).sum())
    return 2 * rows * 32 * 64 * 2 + ctx * KV_BYTES_PER_TOKEN


def host_cpu() -> dict:
    """The host's CPU model and numpy's version, reported with the oracle baseline."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "numpy": np.__version__}


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host's cores, bounded sample
# ---------------------------------------------------------------------------------------
# A one-GPU machine's share of its host is 16 CPUs, whatever the machine shows.
CPU_POOL_MAX = 16
# CPU seconds (workers x wall) the attention baselines aim for.
CPU_TARGET_S = 15.0
_POOL = {}  # inputs of the forked workers (inherited read-only through fork)


def cpu_workers() -> tuple[int, int]:
    """(workers, CPUs this process may run on): one worker per CPU of the affinity set, at
    most CPU_POOL_MAX."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, CPU_POOL_MAX)), n


def _one_blas_thread():
    from threadpoolctl import threadpool_limits

    _POOL["limit"] = threadpool_limits(limits=1)  # kept alive for the worker's lifetime


def _noop(_):
    return 0


def pool_passes(fn, tasks, target_s: float, budget_s: float):
    """Map ``fn`` over ``tasks`` on a fork pool (one BLAS thread per worker), repeating the
    whole pass until the CPU time (workers x wall) reaches ``target_s`` or the wall time
    ``budget_s``.  The workers are started before the clock.  Returns (sum of results,
    passes, wall seconds, workers, affinity CPUs)."""
    import multiprocessing as mp

    workers, aff = cpu_workers()
    with mp.get_context("fork").Pool(workers, initializer=_one_blas_thread) as pool:
        pool.map(_noop, range(workers))
        total, passes = 0, 0
        t0 = time.perf_counter()
        while True:
            total += sum(pool.map(fn, tasks, chunksize=1))
            passes += 1
            wall = time.perf_counter() - t0
            if workers * wall >= target_s or wall >= budget_s:
                break
    return total, passes, wall, workers, aff


def _decode_task(s: int) -> int:
    import oracle as O

    c, kp, vp = _POOL["case"], _POOL["kp"], _POOL["vp"]
    r = c.decode_seqs
    bt = c.block_tables[r.start:r.stop]
    ctx = c.ctx_lens[r.start:r.stop]
    O.decode(c.q_decode, kp, vp, bt, ctx, c.block_size, c.num_kv_heads, c.head_dim, c.scale,
             seqs=[s])
    return int(ctx[s]) * KV_BYTES_PER_TOKEN


def _prefill_task(task) -> int:
    """Rows r0 .. r1 of prefill sequence s: gather its K/V, attend (causal)."""
    import oracle as O

    s, r0, r1 = task
    c, kp, vp = _POOL["case"], _POOL["kp"], _POOL["vp"]
    p = c.prefill_seqs
    seq = p.start + s
    ctx = int(c.ctx_lens[seq])
    cu = c.cu_q_lens_prefill
    qlen = int(cu[s + 1] - cu[s])
    kb, vb = O.gather(kp, vp, c.block_tables[seq], ctx, c.block_size, c.num_kv_heads,
                      c.head_dim)
    vis = [ctx - qlen + i + 1 for i in range(r0, r1)]
    O.attention(O.bf16_to_f64(c.q_prefill[cu[s] + r0:cu[s] + r1]), O.bf16_to_f64(kb),
                O.bf16_to_f64(vb), vis, c.scale)
    return int(sum(vis))


def cpu_baseline(cfg: int, budget_s: float = 20.0) -> dict:
    """The fp64 oracle on layer 0 of workload ``cfg``: decode sequences (gather + three-pass
    softmax) when the workload has them, else the prefill rows, spread over a process
    pool with one worker per host CPU (at most 16) and one BLAS thread each."""
    import oracle as O

    case = W.make_case(cfg, layer=0)
    kp = W.sentinel_pool(case)
    vp = W.sentinel_pool(case)
    O.kv_append(kp, vp, case.k_setup, case.v_setup, case.block_tables, case.cu_setup_lens,
                case.setup_ctx_lens, case.block_size)
    O.kv_append(kp, vp, case.k_new, case.v_new, case.block_tables, case.cu_new_lens,
                case.ctx_lens, case.block_size)
    _POOL.update(case=case, kp=kp, vp=vp)
    r = case.decode_seqs
    try:
        if len(r):
            tasks = list(range(len(r)))
            nbytes, passes, dt, workers, aff = pool_passes(_decode_task, tasks, CPU_TARGET_S,
                                                          budget_s)
            return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": workers,
                    "affinity_cpus": aff, "kind": "oracle",
                    "sample": f"fp64 numpy oracle decode (gather + three-pass softmax) of all "
                              f"{len(r)} decode sequences of layer 0, {passes} pass(es) "
                              f"({nbytes / 1e6:.1f} MB of KV) in {dt:.2f} s on {workers} "
                              f"worker processes, 1 BLAS thread each"}
        p = case.prefill_seqs
        cu = case.cu_q_lens_prefill
        tasks = [(s, r0, min(r0 + 64, int(cu[s + 1] - cu[s])))
                 for s in range(len(p)) for r0 in range(0, int(cu[s + 1] - cu[s]), 64)]
        tasks.sort(key=lambda t: -(t[2] + int(case.ctx_lens[p.start + t[0]])))  # longest first
        pairs, passes, dt, workers, aff = pool_passes(_prefill_task, tasks, CPU_TARGET_S,
                                                      budget_s)
        return {"value": pairs * FLOP_PER_PAIR / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
                "affinity_cpus": aff, "kind": "oracle",
                "sample": f"fp64 numpy oracle causal prefill of all {len(p)} prompts "
                          f"({len(tasks)} blocks of up to 64 rows), {passes} pass(es) in "
                          f"{dt:.2f} s on {workers} worker processes, 1 BLAS thread each"}
    finally:
        _POOL.clear()


# ---------------------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------------------
class Layer:
    """One layer's pools and step inputs on the device."""

    def __init__(self, case: W.Case, torch, pa, bt, ctx, cu_new, cu_q):
        dev = torch.device("cuda:0")

        def up16(bits):
            a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
            return torch.from_numpy(a).to(dev).view(torch.bfloat16)

        e = W.page_elems(case)
        self.kp = torch.zeros((case.num_pages, e), dtype=torch.bfloat16, device=dev)
        self.vp = torch.zeros((case.num_pages, e), dtype=torch.bfloat16, device=dev)
        self.geom = pa.Geometry(case.num_pages, case.block_size, case.num_q_heads,
                                case.num_kv_heads, case.head_dim)
        if case.k_setup.shape[0]:
            ks, vs = up16(case.k_setup), up16(case.v_setup)
            pa.kv_append(self.geom, ks, vs, self.kp, self.vp, bt,
                         torch.from_numpy(case.cu_setup_lens).to(dev),
                         torch.from_numpy(case.setup_ctx_lens).to(dev))
            del ks, vs
        self.k_new = up16(case.k_new)
        self.v_new = up16(case.v_new)
        self.q_dec = up16(case.q_decode) if len(case.decode_seqs) else None
        self.q_pre = up16(case.q_prefill) if len(case.prefill_seqs) else None


class HeadStart:
    """A GPU spin queued ahead of a timed eager step: while it runs, the host enqueues the
    step's launches and events, so the kernels then run back to back and per-launch events
    measure kernel time, not the host's launch rate.  The spin lasts twice the eager step's
    wall time (at least 1 ms), calibrated once against events."""

    def __init__(self, torch, stream, step_s: float):
        self.torch, self.stream = torch, stream
        self.ms = max(1.0, 2e3 * step_s)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        probe = 1 << 20
        with torch.cuda.stream(stream):
            torch.cuda._sleep(probe)  # first call loads the kernel
            a.record(stream)
            torch.cuda._sleep(probe)
            b.record(stream)
        b.synchronize()
        per_ms = probe / max(a.elapsed_time(b), 1e-3)
        self.cycles = int(per_ms * self.ms)

    def __call__(self):
        with self.torch.cuda.stream(self.stream):
            self.torch.cuda._sleep(self.cycles)


def decode_rooflines(res: dict, base: W.Case, traffic_key: str):
    """The line's decode entries: pa_decode against HBM peak, or, when the step ran as one
    pa_decode_append launch per layer, that launch as `roofline` with pa_decode beside it
    as `roofline_decode_only`.  Returns (entries, step_timing additions)."""
    ach = res["decode_gbps"]
    dec_line = {"bound": "hbm",
                "kernel": "pa_decode (decode_stream_kernel + decode_merge_kernel)",
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": hbm_traffic(traffic_key),
                "bytes_per_launch": res["decode_bytes_per_launch"],
                "unique_bytes_per_launch": unique_kv_bytes(base),
                "avg_launch_ms": round(res["decode_ms"], 5)}
    fz = res.get("fused")
    if fz is None:
        return {"roofline": dec_line}, {}
    # the step that value times: one pa_decode_append launch per layer
    extra = {"fused_append": True, "separate_append_graph_ms": round(fz["separate_ms_per_step"], 4),
             "separate_append_value": round(fz["separate_value"], 2)}
    ach = fz["kernel_gbps"]
    fused = {"bound": "hbm",
             "kernel": "pa_decode_append (decode_stream_kernel<bs, append> + decode_merge_kernel)",
             "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBPS, 4), "traffic": hbm_traffic(traffic_key),
             "bytes_per_launch": res["decode_bytes_per_launch"],
             "unique_bytes_per_launch": unique_kv_bytes(base),
             "avg_launch_ms": round(fz["kernel_ms"], 5)}
    dec_line["traffic"] = None  # the counters are taken on the fused launch
    return {"roofline": fused, "roofline_decode_only": dec_line}, extra


def prefill_roofline(res: dict, base: W.Case, traffic_key: str) -> dict:
    """pa_prefill against dense bf16 MFMA peak, and the least HBM traffic the launch needs
    (q and out once, each sequence's K/V once) at the measured time against HBM peak: the
    other bound a prefill launch is near."""
    ach = res["prefill_tflops"]
    min_b = prefill_min_bytes(base)
    gbps = min_b / (res["prefill_ms"] * 1e-3) / 1e9
    return {"bound": "mfma",
            "kernel": "pa_prefill (prefill_kernel [+ prefill_merge_kernel when split])",
            "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": hbm_traffic(traffic_key),
            "flop_per_launch": res["prefill_flop_per_launch"],
            "avg_launch_ms": round(res["prefill_ms"], 5),
            "hbm_min_bytes": min_b, "hbm_min_gbps": round(gbps, 1),
            "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def run_gpu(cfg: int, steps: int, warmup: int, partition: int = 0) -> dict:
    import torch

    import paged_kv_attention_31_amd as pa

    dev = torch.device("cuda:0")
    lib = pa.library()
    n_layers = max(W.NUM_LAYERS[cfg], LAYER_COPIES.get(cfg, 1))
    base = W.make_case(cfg, values=False)
    r_dec, r_pre = base.decode_seqs, base.prefill_seqs
    bt = torch.from_numpy(base.block_tables).to(dev)
    ctx = torch.from_numpy(base.ctx_lens).to(dev)
    cu_new = torch.from_numpy(base.cu_new_lens).to(dev)
    cu_q = torch.from_numpy(base.cu_q_lens_prefill).to(dev)
    dec_bt, dec_ctx = bt[r_dec.start:r_dec.stop], ctx[r_dec.start:r_dec.stop]
    pre_bt, pre_ctx = bt[r_pre.start:r_pre.stop], ctx[r_pre.start:r_pre.stop]
    layers = []
    for li in range(n_layers):
        t0 = time.perf_counter()
        case = W.fill_values(W.make_case(cfg, values=False), li % W.NUM_LAYERS[cfg] if
                             cfg in LAYER_COPIES else li)
        layers.append(Layer(case, torch, pa, bt, ctx, cu_new, cu_q))
        del case
        torch.cuda.synchronize()
        log(f"layer {li} resident ({time.perf_counter() - t0:.1f} s)")
    geom = layers[0].geom
    n_dec, n_pre = len(r_dec), len(r_pre)
    max_ctx_dec = int(base.ctx_lens[r_dec.start:r_dec.stop].max()) if n_dec else 0
    max_ctx_pre = int(base.ctx_lens[r_pre.start:r_pre.stop].max()) if n_pre else 0
    max_q = int(base.q_lens_prefill.max()) if n_pre else 0
    part = pa.decode_partition_tokens(geom, n_dec, max_ctx_dec, partition) if n_dec else 0
    ws_bytes = pa.decode_workspace_bytes(geom, n_dec, max_ctx_dec, part) if n_dec else 0
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    pre_ws_bytes = pa.prefill_workspace_bytes(geom, n_pre, max_q, max_ctx_pre) if n_pre else 0
    pre_ws = torch.empty(max(pre_ws_bytes, 1), dtype=torch.uint8, device=dev)
    out_dec = torch.empty((n_dec, 32, 64), dtype=torch.bfloat16, device=dev)
    out_pre = torch.empty((int(base.q_lens_prefill.sum()), 32, 64), dtype=torch.bfloat16,
                          device=dev)
    stream = torch.cuda.current_stream()
    scale = base.scale

    def launch_append(L, st):
        pa.kv_append(geom, L.k_new, L.v_new, L.kp, L.vp, bt, cu_new, ctx, stream=st)

    def launch_prefill(L, st):
        pa.prefill(geom, out_pre, L.q_pre, L.kp, L.vp, pre_bt, cu_q, pre_ctx, max_q,
                   max_ctx_pre, scale, causal=True, workspace=pre_ws, stream=st)

    def launch_decode(L, st):
        pa.decode(geom, out_dec, L.q_dec, L.kp, L.vp, dec_bt, dec_ctx, max_ctx_dec,
                  scale, partition_tokens=part, workspace=ws, stream=st)

    def step(stream):
        for L in layers:
            launch_append(L, stream)
            if n_pre:
                launch_prefill(L, stream)
            if n_dec:
                launch_decode(L, stream)

    for _ in range(warmup):
        step(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step(stream)
    host_s = time.perf_counter() - t0  # host enqueue time of a step (an upper bound)
    torch.cuda.synchronize()
    log(f"timing {steps} eager steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0
    # Per-kernel times: HIP events around a batch of one kernel's launches, one per layer
    # (each launch repeats the step's own work: the append rewrites the same rows, prefill
    # and decode only read the pools), queued behind a GPU spin that outlasts the host's
    # enqueueing, so the launches run back to back and the events time the GPU alone.
    # Events around single launches are not used: on this runtime they can read several
    # times the kernel's duration when the host falls behind.
    # A batch holds at least 16 launches (the layer loop repeated for workloads of few
    # layers) so the first launch's start-up is spread over many.
    reps = max(1, -(-16 // n_layers))
    hold = HeadStart(torch, stream, host_s * reps)
    kinds = [("append", launch_append)] + ([("prefill", launch_prefill)] if n_pre else []) + \
        ([("decode", launch_decode)] if n_dec else [])
    ev = {k: [] for k, _ in kinds}
    log(f"timing {steps} batches of each kernel ({hold.ms:.1f} ms head start)")
    for _ in range(steps):
        hold()
        for k, fn in kinds:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _r in range(reps):
                for L in layers:
                    fn(L, stream)
            b.record(stream)
            ev[k].append((a, b))
    torch.cuda.synchronize()
    # whole-step time: the same step captured once in a HIP graph and replayed, which
    # removes the host launch gaps between the 16 x 3 launches
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.graph(graph, stream=cap):
        step(cap)
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    log(f"timing {steps} graph replays")
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def avg_ms(pairs):  # per launch: each pair brackets reps launches per layer
        return float(np.mean([a.elapsed_time(b) for a, b in pairs])) / (n_layers * reps) if pairs else 0.0

    # A pure decode step (one new token per sequence, no prefill) also runs as one
    # pa_decode_append launch per layer: timed per launch (events) and as a graph, and
    # that step gives the value.
    fused = None
    if n_dec and not n_pre and int(base.cu_new_lens[-1]) == n_dec:
        hkv = base.num_kv_heads

        def fused_step(st):
            for L in layers:
                pa.decode_append(geom, out_dec, L.q_dec, L.k_new.view(n_dec, hkv, 64),
                                 L.v_new.view(n_dec, hkv, 64), L.kp, L.vp, dec_bt, dec_ctx,
                                 max_ctx_dec, scale, partition_tokens=part, workspace=ws,
                                 stream=st)

        ev_fused = []
        for _ in range(warmup):
            fused_step(stream)
        torch.cuda.synchronize()
        for _ in range(steps):  # a batch of reps launches per layer, as above
            hold()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _r in range(reps):
                fused_step(stream)
            b.record(stream)
            ev_fused.append((a, b))
        torch.cuda.synchronize()
        graph_f = torch.cuda.CUDAGraph()
        cap_f = torch.cuda.Stream()
        cap_f.wait_stream(stream)
        with torch.cuda.graph(graph_f, stream=cap_f):
            fused_step(cap_f)
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph_f.replay()
        torch.cuda.synchronize()
        log(f"timing {steps} graph replays of the fused step")
        t0 = time.perf_counter()
        for _ in range(steps):
            graph_f.replay()
        torch.cuda.synchronize()
        fused = {"ms_per_step": (time.perf_counter() - t0) * 1e3 / steps,
                 "kernel_ms": avg_ms(ev_fused)}

    ms_step = wall * 1e3 / steps
    res = {"ms_per_step": ms_step, "ms_per_step_eager": wall_eager * 1e3 / steps,
           "n_layers": n_layers, "partition_tokens": part, "append_ms": avg_ms(ev["append"]),
           "fused": fused}
    kv_bytes_layer = base.kv_tokens() * KV_BYTES_PER_TOKEN
    if n_dec:
        dec_ms = avg_ms(ev["decode"])
        res.update(decode_ms=dec_ms, decode_bytes_per_launch=kv_bytes_layer,
                   decode_gbps=kv_bytes_layer / (dec_ms * 1e-3) / 1e9,
                   value=kv_bytes_layer * n_layers / (ms_step * 1e-3) / 1e9, unit="GB/s")
        if fused is not None:
            fused.update(value=kv_bytes_layer * n_layers / (fused["ms_per_step"] * 1e-3) / 1e9,
                         kernel_gbps=kv_bytes_layer / (fused["kernel_ms"] * 1e-3) / 1e9,
                         separate_value=res["value"], separate_ms_per_step=ms_step)
            res.update(value=fused["value"], ms_per_step=fused["ms_per_step"])
    if n_pre:
        pre_ms = avg_ms(ev["prefill"])
        flops = base.prefill_pairs() * FLOP_PER_PAIR
        res.update(prefill_ms=pre_ms, prefill_flop_per_launch=flops,
                   prefill_tflops=flops / (pre_ms * 1e-3) / 1e12)
        if not n_dec:
            res.update(value=flops * n_layers / (ms_step * 1e-3) / 1e12, unit="TFLOP/s")
    res["lib"] = os.path.basename(pa._lib.LIB_PATH)
    del lib
    return res


def n_copies(footprint: int) -> int:
    """Independent buffer sets a kernel-level workload rotates over (at least two)."""
    return max(2, -(-ROTATE_BYTES // max(footprint, 1)))


def timed_rotating(fns, steps: int, stream) -> float:
    """Average HIP-event time of one launch over ``steps`` launches that cycle through
    ``fns`` (one closure per buffer set): events around batches of 16 back-to-back launches,
    each batch queued behind a head start (``HeadStart``) so that none of them waits for the
    host."""
    import torch

    t0 = time.perf_counter()
    for fn in fns:
        fn()
    host_s = (time.perf_counter() - t0) / len(fns)  # host enqueue time per launch (upper bound)
    torch.cuda.synchronize()
    chunk = 16
    hold = HeadStart(torch, stream, host_s * chunk)
    ev, i = [], 0
    while i < steps:
        n = min(chunk, steps - i)
        hold()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for k in range(n):
            fns[(i + k) % len(fns)]()
        b.record(stream)
        ev.append((a, b, n))
        i += n
    torch.cuda.synchronize()
    return float(sum(x.elapsed_time(y) for x, y, _ in ev) / sum(n for _, _, n in ev))


def run_rope(cfg: int, steps: int, warmup: int) -> dict:
    """pa_rope_kv_append over the new rows of workload ``cfg`` (one layer), timed with HIP
    events per launch; pa_kv_append of the same rows timed the same way beside it."""
    import torch

    import paged_kv_attention_31_amd as pa

    dev = torch.device("cuda:0")
    case = W.make_case(cfg)
    stream = torch.cuda.current_stream()

    def up16(bits):
        a = np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)
        return torch.from_numpy(a).to(dev).view(torch.bfloat16)

    geom = pa.Geometry(case.num_pages, case.block_size, case.num_q_heads, case.num_kv_heads,
                       case.head_dim)
    e = W.page_elems(case)
    bt = torch.from_numpy(case.block_tables).to(dev)
    ctx = torch.from_numpy(case.ctx_lens).to(dev)
    cu = torch.from_numpy(case.cu_new_lens).to(dev)
    k0, v0 = up16(case.k_new), up16(case.v_new)
    t = int(case.k_new.shape[0])
    q0 = up16(W.normal_bf16([77, cfg], t * case.num_q_heads * case.head_dim)).view(
        t, case.num_q_heads, case.head_dim)
    row = case.num_kv_heads * case.head_dim * 2  # bytes of one token's K (or V) row
    qrow = case.num_q_heads * case.head_dim * 2
    footprint = 2 * case.num_pages * e * 2 + t * (2 * qrow + 2 * row)
    ropes, plains = [], []
    for _ in range(n_copies(footprint)):
        kp = torch.zeros((case.num_pages, e), dtype=torch.bfloat16, device=dev)
        vp = torch.zeros_like(kp)
        q, k_new, v_new = q0.clone(), k0.clone(), v0.clone()
        q_out = torch.empty_like(q)
        ropes.append(lambda q=q, q_out=q_out, k_new=k_new, v_new=v_new, kp=kp, vp=vp:
                     pa.rope_kv_append(geom, q, q_out, k_new, v_new, kp, vp, bt, cu, ctx,
                                       rope_theta=500000.0, stream=stream))
        plains.append(lambda k_new=k_new, v_new=v_new, kp=kp, vp=vp:
                      pa.kv_append(geom, k_new, v_new, kp, vp, bt, cu, ctx, stream=stream))
    for _ in range(warmup):
        ropes[0]()
        plains[0]()
    torch.cuda.synchronize()
    rope_ms = timed_rotating(ropes, steps, stream)
    plain_ms = timed_rotating(plains, steps, stream)
    nbytes = t * (2 * qrow + 4 * row)  # q read + written, K/V read + written
    return {"rope_ms": rope_ms, "plain_ms": plain_ms, "bytes_per_launch": nbytes,
            "plain_bytes_per_launch": t * 4 * row, "tokens": t, "ms_per_step": rope_ms,
            "buffer_sets": len(ropes),
            "gbps": nbytes / (rope_ms * 1e-3) / 1e9,
            "plain_gbps": t * 4 * row / (plain_ms * 1e-3) / 1e9}


def copy_calibration(nbytes: int, reps: int) -> dict:
    """Device-to-device copy of ``nbytes`` (torch's copy kernel), timed with HIP events.

    Gives the box's achievable HBM bandwidth as context, and a kernel whose HBM traffic
    is known exactly (nbytes read + nbytes written per launch), against which the
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters are scaled."""
    import torch

    dev = torch.device("cuda:0")
    n = nbytes // 2
    a = torch.empty(n, dtype=torch.int16, device=dev).fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ms = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        b.copy_(a)
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    avg = float(np.mean(ms[1:] if len(ms) > 1 else ms))
    return {"kind": "hbm-copy", "bytes_read": 2 * n, "bytes_written": 2 * n, "reps": reps,
            "avg_ms": round(avg, 5),
            "gbps_read_plus_write": round(4 * n / (avg * 1e-3) / 1e9, 1)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixed", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill-target", action="store_true",
                    help="mixed workload: skip the 8-prompt prefill measurement")
    ap.add_argument("--no-decode-targets", action="store_true",
                    help="mixed workload: skip the batched and long-context decode measurements")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--partition", type=int, default=0,
                    help="decode KV tokens per split-K partition (0 = the library's choice)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the workload, time a device copy of this many bytes "
                         "(HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the library has no "
              "multi-GPU path; the attention shards by sequence or KV head with no exchange",
              file=sys.stderr)
        return 2
    if args.copy_bytes > 0:
        print(json.dumps(copy_calibration(args.copy_bytes, max(2, args.steps))), flush=True)
        return 0
    cfg = WORKLOADS[args.workload]
    if args.workload == "rope-append":
        return main_rope(args, cfg)
    if args.workload == "copy-pages":
        return main_copy(args)
    if args.workload == "norm-mlp":
        return main_norm(args)
    if args.workload == "serve":
        return main_serve(args)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(cfg, args.cpu_budget)
        log(f"cpu baseline: {cpu['value']:.4f} {cpu['unit']}")

    res = run_gpu(cfg, args.steps, args.warmup, args.partition)
    base = W.make_case(cfg, values=False)
    config = {"workload": W.CONFIG_NAMES[cfg], "layers": res["n_layers"],
              "block_size": base.block_size, "num_q_heads": 32, "num_kv_heads": 8,
              "head_dim": 64, "decode_seqs": len(base.decode_seqs),
              "prefill_seqs": len(base.prefill_seqs),
              "decode_kv_tokens_per_layer": base.kv_tokens(),
              "prefill_visible_pairs_per_layer": base.prefill_pairs(),
              "partition_tokens": res["partition_tokens"]}
    line = {
        "metric": METRIC,
        "value": round(res["value"], 2),
        "unit": res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/Q, shuffled pages)",
        "config": config,
        "step_timing": {"graph_replay_ms": round(res["ms_per_step"], 4),
                        "eager_ms": round(res["ms_per_step_eager"], 4)},
    }
    if "decode_ms" in res:
        rl, extra = decode_rooflines(res, base, args.workload)
        line.update(rl)
        line["step_timing"].update(extra)
    if "prefill_ms" in res:
        key = "roofline_prefill" if "roofline" in line else "roofline"
        line[key] = prefill_roofline(res, base, args.workload + "-prefill"
                                     if key == "roofline_prefill" else args.workload)
    if args.workload == "mixed" and not args.no_prefill_target:
        # the prefill target's own workload (8 whole prompts), measured in the same run
        log("prefill workload (8 prompts) for the prefill roofline")
        res3 = run_gpu(3, args.steps, args.warmup)
        base3 = W.make_case(3, values=False)
        line["roofline_prefill_8prompts"] = dict(
            {"workload": W.CONFIG_NAMES[3], "layer_copies": res3["n_layers"]},
            **prefill_roofline(res3, base3, "prefill"))
    if args.workload == "mixed" and not args.no_decode_targets:
        # the pure decode workloads (64 sequences of up to 2k tokens; 16 x 32k tokens), each
        # run as its own step of pa_decode_append launches, measured in the same run
        for wl in ("decode-batched", "decode-long"):
            log(f"{wl} workload for its decode roofline")
            cfg_d = WORKLOADS[wl]
            res_d = run_gpu(cfg_d, args.steps, args.warmup)
            base_d = W.make_case(cfg_d, values=False)
            rl, _ = decode_rooflines(res_d, base_d, wl)
            line[f"roofline_{wl.replace('-', '_')}"] = dict(
                {"workload": W.CONFIG_NAMES[cfg_d], "layer_copies": res_d["n_layers"],
                 "step_value": round(res_d["value"], 2), "step_ms": round(res_d["ms_per_step"], 4)},
                **{k.replace("roofline", "launch"): v for k, v in rl.items()})
    line["append_ms_per_layer"] = round(res["append_ms"], 5)
    line["cpu_baseline"] = dict(cpu, **host_cpu()) if cpu else cpu
    print(json.dumps(line), flush=True)
    return 0


def run_copy(steps: int, warmup: int) -> dict:
    """pa_copy_pages of COPY_PAGES pages onto as many others, both pools, HIP-event timed."""
    import torch

    import paged_kv_attention_31_amd as pa

    dev = torch.device("cuda:0")
    n_pages = 2 * COPY_PAGES
    e = COPY_BS * 8 * 64
    pools = [(torch.empty((n_pages, e), dtype=torch.bfloat16, device=dev).normal_(),
              torch.empty((n_pages, e), dtype=torch.bfloat16, device=dev).normal_())
             for _ in range(n_copies(2 * n_pages * e * 2))]
    perm = np.random.default_rng(7).permutation(n_pages).astype(np.int32)
    src = torch.from_numpy(perm[:COPY_PAGES].copy()).to(dev)
    dst = torch.from_numpy(perm[COPY_PAGES:].copy()).to(dev)
    geom = pa.Geometry(n_pages, COPY_BS, 32, 8, 64)
    stream = torch.cuda.current_stream()
    fns = [lambda kp=kp, vp=vp: pa.copy_pages(geom, kp, vp, src, dst, stream=stream)
           for kp, vp in pools]
    for _ in range(warmup):
        fns[0]()
    torch.cuda.synchronize()
    ms = timed_rotating(fns, steps, stream)
    nbytes = COPY_PAGES * e * 2 * 2 * 2  # both pools, read + written
    return {"ms": ms, "bytes_per_launch": nbytes, "gbps": nbytes / (ms * 1e-3) / 1e9,
            "ms_per_step": ms, "buffer_sets": len(fns)}


def _copy_task(j: int) -> int:
    import oracle as O

    kp, vp, perm, blk = _POOL["kp"], _POOL["vp"], _POOL["perm"], _POOL["blk"]
    n = len(perm) // 2
    src, dst = perm[j * blk:(j + 1) * blk], perm[n + j * blk:n + (j + 1) * blk]
    O.copy_pages(kp, vp, src, dst)
    return len(src) * kp.shape[1] * 2 * 2 * 2  # both pools, read and written


def cpu_baseline_copy(budget_s: float) -> dict:
    """The oracle's page copies (numpy) on a bounded sample of pairs of the same size,
    blocks of pairs spread over a process pool (one worker per host CPU, at most 16)."""
    e = COPY_BS * 8 * 64
    n = 512  # pages per pool in the sample (the oracle holds both pools in host memory)
    kp = np.random.default_rng(1).integers(0, 1 << 16, (2 * n, e), dtype=np.uint16)
    _POOL.update(kp=kp, vp=kp.copy(), perm=np.random.default_rng(7).permutation(2 * n), blk=32)
    try:
        nbytes, passes, dt, workers, aff = pool_passes(_copy_task, list(range(n // 32)),
                                                      min(CPU_TARGET_S, 5.0), min(budget_s, 5.0))
    finally:
        _POOL.clear()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": workers, "affinity_cpus": aff,
            "kind": "oracle",
            "sample": f"numpy oracle copy of {n} block-size-32 page pairs (blocks of 32 pairs, "
                      f"each worker on its own copy of the pools) x {passes} in {dt:.2f} s on "
                      f"{workers} worker processes"}


def main_copy(args) -> int:
    cpu = None if args.no_cpu_baseline else cpu_baseline_copy(args.cpu_budget)
    res = run_copy(args.steps, args.warmup)
    line = {
        "metric": METRIC, "value": round(res["gbps"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) bf16 pools, seeded page permutation)",
        "config": {"workload": f"copy-pages-{COPY_PAGES}x-bs{COPY_BS}", "layers": 1,
                   "block_size": COPY_BS, "num_kv_heads": 8, "head_dim": 64,
                   "buffer_sets": res["buffer_sets"]},
        "roofline": {"bound": "hbm", "kernel": "pa_copy_pages (copy_pages_kernel)",
                     "achieved": round(res["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(res["gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": hbm_traffic("copy-pages"),
                     "bytes_per_launch": res["bytes_per_launch"],
                     "avg_launch_ms": round(res["ms"], 5)},
        "cpu_baseline": dict(cpu, **host_cpu()) if cpu else cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def run_norm(steps: int, warmup: int) -> dict:
    """pa_silu_mul and pa_residual_rmsnorm at the 1B shape, HIP-event timed per launch."""
    import torch

    import paged_kv_attention_31_amd as pa

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    silu_bytes = NORM_ROWS * MLP_WIDTH * 2 * 3      # gate, up read; product written
    norm_bytes = NORM_ROWS * HIDDEN * 2 * 4         # x, residual read; residual, out written
    silus, norms = [], []
    for _ in range(n_copies(silu_bytes)):
        gu = torch.empty((NORM_ROWS, 2 * MLP_WIDTH), dtype=torch.bfloat16, device=dev).normal_()
        act = torch.empty((NORM_ROWS, MLP_WIDTH), dtype=torch.bfloat16, device=dev)
        silus.append(lambda gu=gu, act=act: pa.silu_mul(gu[:, :MLP_WIDTH], gu[:, MLP_WIDTH:], act,
                                                        stream=stream))
    gamma = torch.empty(HIDDEN, dtype=torch.bfloat16, device=dev).normal_()
    for _ in range(n_copies(norm_bytes - NORM_ROWS * HIDDEN * 2)):
        x = torch.empty((NORM_ROWS, HIDDEN), dtype=torch.bfloat16, device=dev).normal_()
        res = torch.empty_like(x).normal_()
        out = torch.empty_like(x)
        norms.append(lambda x=x, res=res, out=out: pa.residual_rmsnorm(
            x, gamma, out, residual_in=res, residual_out=res, stream=stream))

    for _ in range(warmup):
        silus[0]()
        norms[0]()
    silu_ms = timed_rotating(silus, steps, stream)
    norm_ms = timed_rotating(norms, steps, stream)
    return {"silu_ms": silu_ms, "silu_bytes": silu_bytes,
            "silu_gbps": silu_bytes / (silu_ms * 1e-3) / 1e9, "norm_ms": norm_ms,
            "norm_bytes": norm_bytes, "norm_gbps": norm_bytes / (norm_ms * 1e-3) / 1e9,
            "ms_per_step": silu_ms, "buffer_sets": [len(silus), len(norms)]}


def _silu_task(j: int) -> int:
    import oracle as O

    g, u = _POOL["g"], _POOL["u"]
    O.silu_mul(g[8 * j:8 * j + 8], u[8 * j:8 * j + 8])
    return 8 * MLP_WIDTH * 6


def cpu_baseline_norm(budget_s: float) -> dict:
    """The oracle's SiLU product on a bounded slice of rows of the same shape, blocks of 8
    rows spread over a process pool (one worker per host CPU, at most 16)."""
    rows = 128
    _POOL.update(g=W.normal_bf16([72, 0], rows * MLP_WIDTH).reshape(rows, MLP_WIDTH),
                 u=W.normal_bf16([72, 1], rows * MLP_WIDTH).reshape(rows, MLP_WIDTH))
    try:
        nbytes, passes, dt, workers, aff = pool_passes(_silu_task, list(range(rows // 8)),
                                                      min(CPU_TARGET_S, 5.0), min(budget_s, 5.0))
    finally:
        _POOL.clear()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": workers, "affinity_cpus": aff,
            "kind": "oracle",
            "sample": f"fp64 numpy silu(g) * u oracle on {rows} x {MLP_WIDTH} x {passes} in "
                      f"{dt:.2f} s on {workers} worker processes, 1 BLAS thread each"}


def serve_stream():
    rng = np.random.default_rng([93, 0])
    return (rng.integers(128, 1025, SERVE_REQS).tolist(), rng.integers(16, 129, SERVE_REQS).tolist())


def run_serve() -> dict:
    """The slot scheduler (pa_sched_step) driving pa_kv_append + pa_prefill / pa_decode on
    each of SERVE_LAYERS layers over SERVE_REQS requests until all have finished: every
    plan is uploaded once and run as is.
    The stream runs twice: once for the wall time and the scheduler's own host time, once
    with each step's kernels timed by HIP events around their batch."""
    import torch

    import paged_kv_attention_31_amd as pa

    dev = torch.device("cuda:0")
    prompts, news = serve_stream()
    max_blocks = -(-(1024 + 128 - 1) // SERVE_BS)
    n_pages = int(SERVE_SLOTS * max_blocks * 1.1)
    geom = pa.Geometry(n_pages, SERVE_BS, 32, 8, 64)
    e = SERVE_BS * 8 * 64
    pools = [(torch.empty((n_pages, e), dtype=torch.bfloat16, device=dev).normal_(),
              torch.empty((n_pages, e), dtype=torch.bfloat16, device=dev).normal_())
             for _ in range(SERVE_LAYERS)]
    rows_max = max(SERVE_CHUNK, SERVE_SLOTS)
    k_src = torch.empty((rows_max, 8, 64), dtype=torch.bfloat16, device=dev).normal_()
    v_src = torch.empty_like(k_src).normal_()
    q_src = torch.empty((rows_max, 32, 64), dtype=torch.bfloat16, device=dev).normal_()
    out = torch.empty_like(q_src)
    stream = torch.cuda.current_stream()

    def serve_pass(hold=None):
        """Run the request stream through a fresh pool and scheduler.  With ``hold`` the
        kernels of each step (one launch per layer) are timed as one batch between HIP
        events, queued behind that head start; a prefill step's appends run before it."""
        pool = pa.PagePool(n_pages)
        sched = pa.Scheduler(pool, SERVE_SLOTS, SERVE_BS, max_blocks, SERVE_CHUNK)
        for rid, (p, m) in enumerate(zip(prompts, news)):
            sched.submit(rid, p, m)
        ev = {pa.STEP_PREFILL: [], pa.STEP_DECODE: []}
        kv_bytes = pairs = 0
        n_steps = {pa.STEP_PREFILL: 0, pa.STEP_DECODE: 0}
        sched_s, host_s = 0.0, 0.0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while True:
            a = time.perf_counter()
            plan = sched.step()
            sched_s += time.perf_counter() - a
            if plan.kind == pa.STEP_IDLE:
                if sched.pending() == 0:
                    break
                continue
            n = len(plan.req_ids)
            t = int(plan.cu_new_lens[-1])
            bt = torch.from_numpy(plan.block_tables).to(dev)
            ctx = torch.from_numpy(plan.ctx_lens).to(dev)
            cu = torch.from_numpy(plan.cu_new_lens).to(dev)
            if plan.kind == pa.STEP_PREFILL:  # one block table serves every layer
                for kp, vp in pools:
                    pa.kv_append(geom, k_src[:t], v_src[:t], kp, vp, bt, cu, ctx, stream=stream)
            if hold is not None:
                hold()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            a = time.perf_counter()
            for kp, vp in pools:
                if plan.kind == pa.STEP_PREFILL:
                    pa.prefill(geom, out[:t], q_src[:t], kp, vp, bt, cu, ctx, plan.max_new_len,
                               plan.max_ctx_len, 0.125, causal=True, stream=stream)
                else:  # one new token per row: append and attend in one launch
                    pa.decode_append(geom, out[:n], q_src[:n], k_src[:n], v_src[:n], kp, vp, bt,
                                     ctx, plan.max_ctx_len, 0.125, stream=stream)
            host_s = max(host_s, time.perf_counter() - a)
            if hold is not None:
                e1.record(stream)
                ev[plan.kind].append((e0, e1))
            if plan.kind == pa.STEP_PREFILL:
                lens = np.diff(plan.cu_new_lens).astype(np.int64)
                c = plan.ctx_lens.astype(np.int64)
                pairs += SERVE_LAYERS * int(np.sum(lens * (c - lens) + lens * (lens + 1) // 2))
            else:
                kv_bytes += (SERVE_LAYERS * int(plan.ctx_lens.astype(np.int64).sum())
                             * KV_BYTES_PER_TOKEN)
            n_steps[plan.kind] += 1
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        sched.close()
        return ev, kv_bytes, pairs, n_steps, sched_s, wall, host_s

    # pass 1: wall time and scheduler time, no events; pass 2: the same stream again, each
    # step's kernels timed as one batch behind a head start
    _, kv_bytes, pairs, n_steps, sched_s, wall, host_s = serve_pass()
    ev = serve_pass(HeadStart(torch, stream, host_s))[0]
    dec_ms = sum(x.elapsed_time(y) for x, y in ev[pa.STEP_DECODE])
    pre_ms = sum(x.elapsed_time(y) for x, y in ev[pa.STEP_PREFILL])
    steps = n_steps[pa.STEP_PREFILL] + n_steps[pa.STEP_DECODE]
    return {"wall_s": wall, "steps": steps, "prefill_steps": n_steps[pa.STEP_PREFILL],
            "decode_steps": n_steps[pa.STEP_DECODE], "sched_us_per_step": sched_s * 1e6 / steps,
            "decode_gbps": kv_bytes / (dec_ms * 1e-3) / 1e9, "decode_kv_bytes": kv_bytes,
            "decode_ms": dec_ms, "prefill_ms": pre_ms,
            "prefill_tflops": pairs * FLOP_PER_PAIR / (pre_ms * 1e-3) / 1e12,
            "tokens": int(sum(news)), "prompt_tokens": int(sum(prompts)),
            "ms_per_step": wall * 1e3 / steps}


def _serve_task(ctxs) -> int:
    """The oracle's attention for a block of decode rows of the serve stream (one layer)."""
    import oracle as O

    q, k, v = _POOL["sq"], _POOL["sk"], _POOL["sv"]
    n = 0
    for ctx in ctxs:
        O.attention(q, k[:ctx], v[:ctx], [ctx], 0.125)
        n += ctx * KV_BYTES_PER_TOKEN
    return n


def cpu_baseline_serve(budget_s: float) -> dict:
    """The oracle scheduler over the same request stream (sequential: each step depends on
    the last), then the oracle's attention (fp64, contiguous K/V) for the rows of its decode
    steps, one layer, spread over the process pool in blocks of rows."""
    from oracle import sched as S

    prompts, news = serve_stream()
    max_blocks = -(-(1024 + 128 - 1) // SERVE_BS)
    sc = S.Scheduler(SERVE_SLOTS, SERVE_BS, max_blocks, SERVE_CHUNK,
                     S.Pool(int(SERVE_SLOTS * max_blocks * 1.1)))
    for rid, (p, m) in enumerate(zip(prompts, news)):
        sc.submit(rid, p, m)
    steps = 0
    ctxs = []
    a = time.perf_counter()
    while True:
        plan = sc.step()
        steps += 1
        if plan.kind == S.IDLE and not sc.queue and not sc.active:
            break
        if plan.kind == S.DECODE:
            ctxs.extend(int(ctx) for _, _, ctx, _, _ in plan.rows)
    sched_s = time.perf_counter() - a
    rng = np.random.default_rng(5)
    _POOL.update(sk=rng.standard_normal((1024 + 128, 8, 64)),
                 sv=rng.standard_normal((1024 + 128, 8, 64)),
                 sq=rng.standard_normal((1, 32, 64)))
    tasks = [ctxs[i:i + 64] for i in range(0, len(ctxs), 64)]
    try:
        nbytes, passes, dt, workers, aff = pool_passes(_serve_task, tasks, CPU_TARGET_S, budget_s)
    finally:
        _POOL.clear()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": workers, "affinity_cpus": aff,
            "kind": "oracle",
            "sample": f"oracle scheduler over the whole stream ({steps} steps, "
                      f"{sched_s * 1e6 / steps:.0f} us/step, sequential), then fp64 oracle "
                      f"attention of the {len(ctxs)} rows of its decode steps, one layer, "
                      f"{passes} pass(es) ({nbytes / 1e9:.2f} GB of KV) in {dt:.2f} s on "
                      f"{workers} worker processes, 1 BLAS thread each"}


def main_serve(args) -> int:
    cpu = None if args.no_cpu_baseline else cpu_baseline_serve(min(args.cpu_budget, 10.0))
    res = run_serve()
    line = {
        "metric": METRIC, "value": round(res["decode_gbps"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": res["steps"], "warmup": 0, "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded request lengths; N(0,1) bf16 pools and rows)",
        "config": {"workload": f"serve-{SERVE_REQS}req-{SERVE_SLOTS}slots-bs{SERVE_BS}",
                   "layers": SERVE_LAYERS, "requests": SERVE_REQS, "slots": SERVE_SLOTS,
                   "prefill_chunk": SERVE_CHUNK, "prompt_range": [128, 1024],
                   "new_tokens_range": [16, 128], "block_size": SERVE_BS},
        "roofline": {"bound": "hbm", "kernel": "pa_decode_append over the scheduled decode steps",
                     "achieved": round(res["decode_gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(res["decode_gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_total": res["decode_kv_bytes"],
                     "kernel_ms_total": round(res["decode_ms"], 3)},
        "serve": {"steps": res["steps"], "prefill_steps": res["prefill_steps"],
                  "decode_steps": res["decode_steps"],
                  "sched_us_per_step": round(res["sched_us_per_step"], 2),
                  "generated_tokens": res["tokens"], "prompt_tokens": res["prompt_tokens"],
                  "wall_s": round(res["wall_s"], 3),
                  "generated_tokens_per_s": round(res["tokens"] / res["wall_s"], 1),
                  "prefill_tflops": round(res["prefill_tflops"], 1),
                  "prefill_kernel_ms_total": round(res["prefill_ms"], 3)},
        "cpu_baseline": dict(cpu, **host_cpu()) if cpu else cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main_norm(args) -> int:
    cpu = None if args.no_cpu_baseline else cpu_baseline_norm(args.cpu_budget)
    res = run_norm(args.steps, args.warmup)
    line = {
        "metric": METRIC, "value": round(res["silu_gbps"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (N(0,1) bf16 activations and gamma)",
        "config": {"workload": f"norm-mlp-{NORM_ROWS}x{HIDDEN}-mlp{MLP_WIDTH}", "layers": 1,
                   "rows": NORM_ROWS, "hidden": HIDDEN, "mlp_width": MLP_WIDTH,
                   "buffer_sets": res["buffer_sets"]},
        "roofline": {"bound": "hbm", "kernel": "pa_silu_mul (silu_mul_kernel)",
                     "achieved": round(res["silu_gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(res["silu_gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": hbm_traffic("norm-mlp"), "bytes_per_launch": res["silu_bytes"],
                     "avg_launch_ms": round(res["silu_ms"], 5)},
        "residual_rmsnorm": {"kernel": "pa_residual_rmsnorm (residual_rmsnorm_kernel)",
                             "bytes_per_launch": res["norm_bytes"],
                             "avg_launch_ms": round(res["norm_ms"], 5),
                             "achieved_gbps": round(res["norm_gbps"], 1),
                             "frac": round(res["norm_gbps"] / HBM_PEAK_GBPS, 4)},
        "cpu_baseline": dict(cpu, **host_cpu()) if cpu else cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def _rope_task(s: int) -> int:
    import oracle as O

    c, q, f = _POOL["case"], _POOL["q"], _POOL["f"]
    if "kp" not in _POOL:  # the worker's own pools
        _POOL["kp"], _POOL["vp"] = W.sentinel_pool(c), W.sentinel_pool(c)
    kp, vp = _POOL["kp"], _POOL["vp"]
    a, b = int(c.cu_new_lens[s]), int(c.cu_new_lens[s + 1])
    O.rope_kv_append(q[a:b], c.k_new[a:b], c.v_new[a:b], kp, vp, c.block_tables[s:s + 1],
                     np.array([0, b - a]), c.ctx_lens[s:s + 1], c.block_size, f)
    return (b - a) * (2 * c.num_q_heads + 4 * c.num_kv_heads) * c.head_dim * 2


def cpu_baseline_rope(cfg: int, budget_s: float) -> dict:
    """The RoPE oracle (fp64 rotation + append) on the same rows, one task per sequence,
    spread over a process pool (one worker per host CPU, at most 16)."""
    import oracle as O

    case = W.make_case(cfg)
    t = int(case.k_new.shape[0])
    q = W.normal_bf16([77, cfg], t * case.num_q_heads * case.head_dim).reshape(
        t, case.num_q_heads, case.head_dim)
    _POOL.update(case=case, q=q, f=O.rope_freqs(case.head_dim, 500000.0))
    try:
        nbytes, passes, dt, workers, aff = pool_passes(_rope_task, list(range(case.n_seqs)),
                                                      CPU_TARGET_S, budget_s)
    finally:
        _POOL.clear()
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": workers, "affinity_cpus": aff,
            "kind": "oracle",
            "sample": f"fp64 numpy RoPE + append oracle on all {t} rows x {passes} in {dt:.2f} s "
                      f"on {workers} worker processes, 1 BLAS thread each"}


def main_rope(args, cfg: int) -> int:
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline_rope(cfg, args.cpu_budget)
    res = run_rope(cfg, args.steps, args.warmup)
    base = W.make_case(cfg, values=False)
    line = {
        "metric": METRIC,
        "value": round(res["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, shuffled pages)",
        "config": {"workload": f"rope-append-{res['tokens']}tokens-bs{base.block_size}",
                   "layers": 1, "block_size": base.block_size, "num_q_heads": 32,
                   "num_kv_heads": 8, "head_dim": 64, "rope_theta": 500000.0,
                   "buffer_sets": res["buffer_sets"]},
        "roofline": {"bound": "hbm", "kernel": "pa_rope_kv_append (append_kernel<bs, rope>)",
                     "achieved": round(res["gbps"], 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(res["gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": hbm_traffic("rope-append"),
                     "bytes_per_launch": res["bytes_per_launch"],
                     "avg_launch_ms": round(res["rope_ms"], 5)},
        "plain_append": {"kernel": "pa_kv_append", "bytes_per_launch": res["plain_bytes_per_launch"],
                         "avg_launch_ms": round(res["plain_ms"], 5),
                         "achieved_gbps": round(res["plain_gbps"], 1)},
        "cpu_baseline": dict(cpu, **host_cpu()) if cpu else cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

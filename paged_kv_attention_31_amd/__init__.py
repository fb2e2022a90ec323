"""paged_kv_attention_31_amd -- paged KV attention for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libpagedattn.so`` (``include/pa.h``).  It only
marshals arguments: PyTorch tensors supply device memory and the current HIP stream,
and every step of the computation runs in the library's HIP kernels.  There is no
fallback: if the library has not been built, every call raises.

Layout (per layer; bf16 = torch.bfloat16):
    k_pool  [num_pages, page_elems]  page = [Hkv][head_dim/8][block_size][8]
    v_pool  [num_pages, page_elems]  page = [Hkv][head_dim][block_size]
    block_tables int32 [n_seqs, max_blocks]; ctx_lens int32 [n_seqs]
    q / out / k_new / v_new: token-major [tokens, heads, head_dim] bf16
"""

from __future__ import annotations

import ctypes
import dataclasses
from typing import NamedTuple, Optional, Sequence

import numpy as np

from . import _lib

__all__ = [
    "PagedAttnError", "Geometry", "PagePool", "Scheduler", "StepPlan", "STEP_IDLE",
    "STEP_PREFILL", "STEP_DECODE", "page_bytes", "kv_append", "rope_kv_append",
    "copy_pages", "residual_rmsnorm", "silu_mul",
    "decode_partition_tokens", "decode_workspace_bytes", "decode", "decode_append",
    "decode_noalloc", "DECODE_SCRATCH_BYTES",
    "prefill_workspace_bytes",
    "prefill", "library",
]


class PagedAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = _lib.load()
        msg = lib.pa_status_string(status).decode()
        if status == _lib.PA_ERR_HIP:
            msg += f" (hipError {lib.pa_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")
        self.status = status


def library():
    """The loaded ctypes library (raises if it was not built)."""
    return _lib.load()


def _check(status: int, where: str) -> None:
    if status != _lib.PA_OK:
        raise PagedAttnError(status, where)


@dataclasses.dataclass(frozen=True)
class Geometry:
    num_pages: int
    block_size: int
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 64

    def c(self) -> _lib.PaGeom:
        return _lib.PaGeom(self.num_pages, self.block_size, self.num_q_heads, self.num_kv_heads,
                           self.head_dim)

    @property
    def page_elems(self) -> int:
        return self.block_size * self.num_kv_heads * self.head_dim


def page_bytes(geom: Geometry) -> int:
    return int(_lib.load().pa_page_bytes(geom.c()))


# ---------------------------------------------------------------------------------------
# host page pool
# ---------------------------------------------------------------------------------------
class PagePool:
    """Free-page list with reference counts (host metadata only)."""

    def __init__(self, num_pages: int):
        self._lib = _lib.load()
        h = ctypes.c_void_p()
        _check(self._lib.pa_pool_create(int(num_pages), ctypes.byref(h)), "pa_pool_create")
        self._h = h

    def close(self) -> None:
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _ids(ids: Sequence[int]):
        arr = (ctypes.c_int32 * len(ids))(*[int(i) for i in ids])
        return arr

    def alloc(self, n: int) -> list[int]:
        out = (ctypes.c_int32 * max(1, n))()
        _check(self._lib.pa_pool_alloc(self._h, int(n), out), "pa_pool_alloc")
        return list(out[:n])

    def share(self, ids: Sequence[int]) -> None:
        _check(self._lib.pa_pool_share(self._h, len(ids), self._ids(ids)), "pa_pool_share")

    def free(self, ids: Sequence[int]) -> None:
        _check(self._lib.pa_pool_free(self._h, len(ids), self._ids(ids)), "pa_pool_free")

    def cow(self, ids: Sequence[int]) -> list[int]:
        """Copy-on-write decision for pages about to be written (see pa_pool_cow): the
        page each entry should write, a fresh one where the original is shared."""
        out = (ctypes.c_int32 * max(1, len(ids)))()
        _check(self._lib.pa_pool_cow(self._h, len(ids), self._ids(ids), out), "pa_pool_cow")
        return list(out[:len(ids)])

    def num_free(self) -> int:
        return int(self._lib.pa_pool_num_free(self._h))

    def refcount(self, page: int) -> int:
        return int(self._lib.pa_pool_refcount(self._h, int(page)))


STEP_IDLE, STEP_PREFILL, STEP_DECODE = _lib.PA_STEP_IDLE, _lib.PA_STEP_PREFILL, _lib.PA_STEP_DECODE


class StepPlan(NamedTuple):
    """One scheduler step (see pa_sched_step): host numpy arrays, row k = request
    req_ids[k] in slot slots[k]."""

    kind: int
    req_ids: np.ndarray       # int64 [n]
    slots: np.ndarray         # int32 [n]
    block_tables: np.ndarray  # int32 [n, max_blocks_per_seq], -1 past the used pages
    ctx_lens: np.ndarray      # int32 [n]
    cu_new_lens: np.ndarray   # int32 [n + 1]
    max_ctx_len: int
    max_new_len: int
    finished: np.ndarray      # int64 ids retired at the start of the step


class Scheduler:
    """Slot scheduler over a PagePool (see pa_sched_*): host decisions only."""

    def __init__(self, pool: PagePool, num_slots: int, block_size: int,
                 max_blocks_per_seq: int, prefill_chunk: int):
        self._lib = _lib.load()
        self._pool = pool  # the pool must outlive the scheduler
        h = ctypes.c_void_p()
        _check(self._lib.pa_sched_create(pool._h, int(num_slots), int(block_size),
                                         int(max_blocks_per_seq), int(prefill_chunk),
                                         ctypes.byref(h)), "pa_sched_create")
        self._h = h
        self.num_slots, self.max_blocks = int(num_slots), int(max_blocks_per_seq)
        self._req = np.zeros(self.num_slots, np.int64)
        self._slots = np.zeros(self.num_slots, np.int32)
        self._bt = np.zeros((self.num_slots, self.max_blocks), np.int32)
        self._ctx = np.zeros(self.num_slots, np.int32)
        self._cu = np.zeros(self.num_slots + 1, np.int32)
        self._fin = np.zeros(self.num_slots, np.int64)

    def close(self) -> None:
        if self._h:
            self._lib.pa_sched_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def submit(self, req_id: int, prompt_len: int, max_new_tokens: int) -> None:
        _check(self._lib.pa_sched_submit(self._h, int(req_id), int(prompt_len),
                                         int(max_new_tokens)), "pa_sched_submit")

    def finish(self, req_id: int) -> None:
        _check(self._lib.pa_sched_finish(self._h, int(req_id)), "pa_sched_finish")

    def pending(self) -> int:
        return int(self._lib.pa_sched_pending(self._h))

    def step(self) -> StepPlan:
        info = _lib.PaSchedStep()
        p = lambda a: a.ctypes.data
        _check(self._lib.pa_sched_step(self._h, ctypes.byref(info), p(self._req), p(self._slots),
                                       p(self._bt), p(self._ctx), p(self._cu), p(self._fin)),
               "pa_sched_step")
        n = int(info.n_seqs)
        return StepPlan(int(info.kind), self._req[:n].copy(), self._slots[:n].copy(),
                        self._bt[:n].copy(), self._ctx[:n].copy(), self._cu[:n + 1].copy(),
                        int(info.max_ctx_len), int(info.max_new_len),
                        self._fin[:int(info.n_finished)].copy())


# ---------------------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------------------
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _scratch(need: int, device, stream):
    """A uint8 workspace of ``need`` bytes allocated here for one call on ``stream``.
    torch's caching allocator ties a block to the stream it was allocated on (the current
    one); when the kernels run on another stream the block is recorded on that stream too,
    so it is not handed out again before the kernels that write it have finished."""
    import torch

    ws = torch.empty(need, dtype=torch.uint8, device=device)
    if stream is not None:
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(
            int(stream), device=device)
        if s.cuda_stream != torch.cuda.current_stream(device).cuda_stream:
            ws.record_stream(s)
    return ws


def _need(cond: bool, what: str) -> None:
    if not cond:
        raise ValueError(what)


def _dev(t, name, dtype, numel=None, dims=None):
    import torch

    _need(t is not None and isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if numel is not None:
        _need(t.numel() == numel, f"{name} has {t.numel()} elements, expected {numel}")
    if dims is not None:
        _need(t.dim() == dims, f"{name} must have {dims} dims")


def kv_append(geom: Geometry, k_new, v_new, k_pool, v_pool, block_tables, cu_new_lens,
              ctx_lens, stream=None) -> None:
    """Write rows ``k_new``/``v_new`` [T, Hkv, d] into the pools (see pa_kv_append)."""
    import torch

    n_seqs = int(ctx_lens.numel())
    t = int(k_new.shape[0]) if k_new.dim() > 0 else 0
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _dev(x, name, torch.bfloat16, t * geom.num_kv_heads * geom.head_dim)
    for name, x in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(x, name, torch.bfloat16, geom.num_pages * geom.page_elems)
    _dev(block_tables, "block_tables", torch.int32, dims=2)
    _dev(cu_new_lens, "cu_new_lens", torch.int32, n_seqs + 1)
    _dev(ctx_lens, "ctx_lens", torch.int32, n_seqs)
    _need(block_tables.shape[0] == n_seqs, "block_tables rows != n_seqs")
    st = _lib.load().pa_kv_append(geom.c(), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                  _ptr(block_tables), int(block_tables.shape[1]),
                                  _ptr(cu_new_lens), _ptr(ctx_lens), n_seqs, t, _stream(stream))
    _check(st, "pa_kv_append")


def copy_pages(geom: Geometry, k_pool, v_pool, src_pages, dst_pages, stream=None) -> None:
    """Copy whole pages src_pages[i] -> dst_pages[i] (int32 device tensors) in both pools
    (see pa_copy_pages)."""
    import torch

    n = int(src_pages.numel())
    for name, x in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(x, name, torch.bfloat16, geom.num_pages * geom.page_elems)
    _dev(src_pages, "src_pages", torch.int32, n)
    _dev(dst_pages, "dst_pages", torch.int32, n)
    st = _lib.load().pa_copy_pages(geom.c(), _ptr(k_pool), _ptr(v_pool), _ptr(src_pages),
                                   _ptr(dst_pages), n, _stream(stream))
    _check(st, "pa_copy_pages")


def residual_rmsnorm(x, gamma, out, residual_in=None, residual_out=None, eps: float = 1e-5,
                     stream=None) -> None:
    """out = RMSNorm(x + residual_in) * gamma per row; the sum goes to residual_out (see
    pa_residual_rmsnorm).  Tensors are bf16 [rows, hidden] (gamma [hidden])."""
    import torch

    _need(x.dim() == 2, "x must be [rows, hidden]")
    rows, hidden = int(x.shape[0]), int(x.shape[1])
    for name, t in (("x", x), ("out", out)):
        _dev(t, name, torch.bfloat16, rows * hidden)
    _dev(gamma, "gamma", torch.bfloat16, hidden)
    _need((residual_in is None) == (residual_out is None),
          "residual_in and residual_out must both be given or both be None")
    if residual_in is not None:
        for name, t in (("residual_in", residual_in), ("residual_out", residual_out)):
            _dev(t, name, torch.bfloat16, rows * hidden)
    st = _lib.load().pa_residual_rmsnorm(_ptr(x), _ptr(residual_in), _ptr(residual_out),
                                         _ptr(gamma), _ptr(out), rows, hidden, float(eps),
                                         _stream(stream))
    _check(st, "pa_residual_rmsnorm")


def silu_mul(gate, up, out, stream=None) -> None:
    """out = silu(gate) * up (see pa_silu_mul).  gate / up / out are bf16 [rows, width]
    views with unit stride along width and equal row strides for gate and up (a
    concatenated gate|up buffer's two halves qualify)."""
    import torch

    _need(gate.dim() == 2 and up.dim() == 2 and out.dim() == 2, "2-d views expected")
    rows, width = int(gate.shape[0]), int(gate.shape[1])
    _need(tuple(up.shape) == (rows, width) and tuple(out.shape) == (rows, width), "shapes differ")
    for name, t in (("gate", gate), ("up", up), ("out", out)):
        _need(t.is_cuda and t.dtype == torch.bfloat16 and t.stride(1) == 1,
              f"{name} must be a bf16 device view with unit inner stride")
    _need(gate.stride(0) == up.stride(0), "gate and up need the same row stride")
    st = _lib.load().pa_silu_mul(_ptr(gate), _ptr(up), int(gate.stride(0)), _ptr(out),
                                 int(out.stride(0)), rows, width, _stream(stream))
    _check(st, "pa_silu_mul")


def rope_kv_append(geom: Geometry, q, q_out, k_new, v_new, k_pool, v_pool, block_tables,
                   cu_new_lens, ctx_lens, rope_theta: float = 500000.0, inv_freq=None,
                   stream=None) -> None:
    """Rotate the new rows' Q (into ``q_out``, which may be ``q``) and K by their
    positions and append K and V to the pools (see pa_rope_kv_append).  ``q``/``q_out``
    may both be None; ``inv_freq`` is None or head_dim/2 float32 frequencies."""
    import torch

    n_seqs = int(ctx_lens.numel())
    t = int(k_new.shape[0]) if k_new.dim() > 0 else 0
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _dev(x, name, torch.bfloat16, t * geom.num_kv_heads * geom.head_dim)
    _need((q is None) == (q_out is None), "q and q_out must both be given or both be None")
    if q is not None:
        for name, x in (("q", q), ("q_out", q_out)):
            _dev(x, name, torch.bfloat16, t * geom.num_q_heads * geom.head_dim)
    if inv_freq is not None:
        _dev(inv_freq, "inv_freq", torch.float32, geom.head_dim // 2)
    for name, x in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(x, name, torch.bfloat16, geom.num_pages * geom.page_elems)
    _dev(block_tables, "block_tables", torch.int32, dims=2)
    _dev(cu_new_lens, "cu_new_lens", torch.int32, n_seqs + 1)
    _dev(ctx_lens, "ctx_lens", torch.int32, n_seqs)
    _need(block_tables.shape[0] == n_seqs, "block_tables rows != n_seqs")
    st = _lib.load().pa_rope_kv_append(
        geom.c(), _ptr(q), _ptr(q_out),
        _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(cu_new_lens), _ptr(ctx_lens), n_seqs, t,
        float(rope_theta), _ptr(inv_freq), _stream(stream))
    _check(st, "pa_rope_kv_append")


def decode_partition_tokens(geom: Geometry, n_seqs: int, max_ctx_len: int,
                            partition_tokens: int = 0) -> int:
    r = int(_lib.load().pa_decode_partition_tokens(geom.c(), n_seqs, max_ctx_len,
                                                    partition_tokens))
    _check(min(r, 0), "pa_decode_partition_tokens")
    return r


def decode_workspace_bytes(geom: Geometry, n_seqs: int, max_ctx_len: int,
                           partition_tokens: int = 0) -> int:
    return int(_lib.load().pa_decode_workspace_bytes(geom.c(), n_seqs, max_ctx_len,
                                                     partition_tokens))


def decode(geom: Geometry, out, q, k_pool, v_pool, block_tables, ctx_lens, max_ctx_len: int,
           scale: float, partition_tokens: int = 0, workspace=None, stream=None) -> None:
    """One query row per sequence over its paged context (see pa_decode).  ``workspace``
    is a uint8 device tensor of at least ``decode_workspace_bytes`` bytes (allocated here
    when omitted)."""
    import torch

    n = int(ctx_lens.numel())
    rows = n * geom.num_q_heads * geom.head_dim
    _dev(out, "out", torch.bfloat16, rows)
    _dev(q, "q", torch.bfloat16, rows)
    for name, x in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(x, name, torch.bfloat16, geom.num_pages * geom.page_elems)
    _dev(block_tables, "block_tables", torch.int32, dims=2)
    _dev(ctx_lens, "ctx_lens", torch.int32, n)
    _need(block_tables.shape[0] == n, "block_tables rows != n_seqs")
    need = decode_workspace_bytes(geom, n, int(max_ctx_len), int(partition_tokens))
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    st = _lib.load().pa_decode(geom.c(), _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                               _ptr(block_tables), int(block_tables.shape[1]), _ptr(ctx_lens), n,
                               int(max_ctx_len), float(scale), int(partition_tokens),
                               _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "pa_decode")


def decode_append(geom: Geometry, out, q, k_new, v_new, k_pool, v_pool, block_tables, ctx_lens,
                  max_ctx_len: int, scale: float, partition_tokens: int = 0, workspace=None,
                  stream=None) -> None:
    """One decode step in one launch (see pa_decode_append): row s of ``k_new`` /
    ``v_new`` [n_seqs, Hkv, d] is appended at position ctx_lens[s] - 1, then the query row
    attends over the whole context.  ``workspace`` as for :func:`decode`."""
    import torch

    n = int(ctx_lens.numel())
    rows = n * geom.num_q_heads * geom.head_dim
    _dev(out, "out", torch.bfloat16, rows)
    _dev(q, "q", torch.bfloat16, rows)
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        _dev(x, name, torch.bfloat16, n * geom.num_kv_heads * geom.head_dim)
    for name, x in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(x, name, torch.bfloat16, geom.num_pages * geom.page_elems)
    _dev(block_tables, "block_tables", torch.int32, dims=2)
    _dev(ctx_lens, "ctx_lens", torch.int32, n)
    _need(block_tables.shape[0] == n, "block_tables rows != n_seqs")
    need = decode_workspace_bytes(geom, n, int(max_ctx_len), int(partition_tokens))
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    st = _lib.load().pa_decode_append(
        geom.c(), _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(ctx_lens), n, int(max_ctx_len),
        float(scale), int(partition_tokens), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "pa_decode_append")


DECODE_SCRATCH_BYTES = _lib.PA_DECODE_SCRATCH_BYTES


def decode_noalloc(geom: Geometry, out, q, k_pool, v_pool, block_tables, ctx_lens,
                   max_ctx_len: int, scale: float, partition_tokens: int = 0,
                   stream=None) -> None:
    """pa_decode without a workspace (see pa_decode_noalloc): the split-K partials go to
    the library's own device scratch of DECODE_SCRATCH_BYTES, so nothing is allocated.
    Calls that overlap on one device share that scratch and must be serialised."""
    import torch

    n = int(ctx_lens.numel())
    rows = n * geom.num_q_heads * geom.head_dim
    _dev(out, "out", torch.bfloat16, rows)
    _dev(q, "q", torch.bfloat16, rows)
    for name, x in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(x, name, torch.bfloat16, geom.num_pages * geom.page_elems)
    _dev(block_tables, "block_tables", torch.int32, dims=2)
    _dev(ctx_lens, "ctx_lens", torch.int32, n)
    _need(block_tables.shape[0] == n, "block_tables rows != n_seqs")
    st = _lib.load().pa_decode_noalloc(geom.c(), _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(block_tables), int(block_tables.shape[1]),
                                       _ptr(ctx_lens), n, int(max_ctx_len), float(scale),
                                       int(partition_tokens), _stream(stream))
    _check(st, "pa_decode_noalloc")


def prefill_workspace_bytes(geom: Geometry, n_seqs: int, max_q_len: int, max_ctx_len: int,
                            kv_splits: int = 0) -> int:
    return int(_lib.load().pa_prefill_workspace_bytes(geom.c(), n_seqs, max_q_len, max_ctx_len,
                                                      kv_splits))


def prefill(geom: Geometry, out, q, k_pool, v_pool, block_tables, cu_q_lens, ctx_lens,
            max_q_len: int, max_ctx_len: int, scale: float, causal: bool = True,
            kv_splits: int = 0, workspace=None, stream=None) -> None:
    """Packed query rows over their sequences' paged contexts (see pa_prefill).
    ``workspace`` is a uint8 device tensor of at least ``prefill_workspace_bytes`` bytes
    (allocated here when omitted)."""
    import torch

    n = int(ctx_lens.numel())
    tq = int(q.shape[0]) if q.dim() > 0 else 0
    rows = tq * geom.num_q_heads * geom.head_dim
    _dev(out, "out", torch.bfloat16, rows)
    _dev(q, "q", torch.bfloat16, rows)
    for name, x in (("k_pool", k_pool), ("v_pool", v_pool)):
        _dev(x, name, torch.bfloat16, geom.num_pages * geom.page_elems)
    _dev(block_tables, "block_tables", torch.int32, dims=2)
    _dev(cu_q_lens, "cu_q_lens", torch.int32, n + 1)
    _dev(ctx_lens, "ctx_lens", torch.int32, n)
    _need(block_tables.shape[0] == n, "block_tables rows != n_seqs")
    need = prefill_workspace_bytes(geom, n, int(max_q_len), int(max_ctx_len), int(kv_splits))
    if workspace is None and need > 0:
        workspace = _scratch(need, q.device, stream)
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    st = _lib.load().pa_prefill(geom.c(), _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_tables), int(block_tables.shape[1]), _ptr(cu_q_lens),
                                _ptr(ctx_lens), n, int(max_q_len), int(max_ctx_len), float(scale),
                                1 if causal else 0, int(kv_splits), _ptr(workspace), ws_bytes,
                                _stream(stream))
    _check(st, "pa_prefill")

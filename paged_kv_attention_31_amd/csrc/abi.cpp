// C ABI of libpagedattn (declared in include/pa.h): argument validation, the host page
// pool, split-K sizing, and dispatch to the HIP launchers.
#include "pa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <vector>

#include "launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  g_last_hip_error = static_cast<int>(e);
  return PA_ERR_HIP;
}

pa::LaunchGeom to_launch(const pa_geom_t& g) {
  return pa::LaunchGeom{g.num_pages, g.block_size, g.num_q_heads, g.num_kv_heads};
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of the current device (the automatic decode plan uses four workers per
// unit); 256 (MI355X) when no device can be queried.
int compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

bool partition_ok(int32_t partition_tokens) {
  return partition_tokens >= 0 && partition_tokens % 64 == 0;
}

// Host-checkable decode arguments shared by the sizing and launch entry points.
int decode_args_ok(const pa_geom_t& g, int32_t n_seqs, int32_t max_ctx_len,
                   int32_t partition_tokens) {
  int st = pa_geom_check(g);
  if (st != PA_OK) return st;
  if (n_seqs < 0 || max_ctx_len < 0 || !partition_ok(partition_tokens)) return PA_ERR_INVALID_ARG;
  // the tile stream is counted in int32 on the device
  const int64_t tiles = std::max<int64_t>(1, ceil_div(max_ctx_len, 64));
  if ((int64_t)n_seqs * tiles * g.num_kv_heads > (int64_t)INT32_MAX) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Host-checkable prefill arguments shared by the sizing and launch entry points.
int prefill_args_ok(const pa_geom_t& g, int32_t n_seqs, int32_t max_q_len, int32_t max_ctx_len,
                    int32_t kv_splits) {
  int st = pa_geom_check(g);
  if (st != PA_OK) return st;
  if (n_seqs < 0 || max_q_len < 0 || max_ctx_len < 0) return PA_ERR_INVALID_ARG;
  if (kv_splits < 0 || kv_splits > pa::kPrefillMaxSplit) return PA_ERR_INVALID_ARG;
  // the grid (tiles x sequences x heads x pieces) must fit one launch dimension
  if (ceil_div(max_q_len, 32) * n_seqs * g.num_kv_heads * pa::kPrefillMaxSplit > (int64_t)INT32_MAX)
    return PA_ERR_INVALID_ARG;
  return PA_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// pool
// ---------------------------------------------------------------------------------------
struct pa_pool {
  std::mutex mu;
  std::vector<int32_t> free_list;  // LIFO stack of free page ids
  std::vector<int32_t> refs;       // reference count per page (0 = free)
};

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_OUT_OF_PAGES: return "out of pages";
    case PA_ERR_UNSUPPORTED: return "unsupported geometry";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int pa_last_hip_error(void) { return g_last_hip_error; }

int pa_version(void) { return 10000; }

int pa_geom_check(pa_geom_t g) {
  if (g.num_pages <= 0 || g.block_size <= 0 || g.num_q_heads <= 0 || g.num_kv_heads <= 0 ||
      g.head_dim <= 0)
    return PA_ERR_INVALID_ARG;
  if (g.head_dim != pa::kHeadDim) return PA_ERR_UNSUPPORTED;
  if (g.block_size != 16 && g.block_size != 32) return PA_ERR_UNSUPPORTED;
  if (g.num_q_heads != pa::kGroup * g.num_kv_heads) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

size_t pa_page_bytes(pa_geom_t g) {
  if (g.block_size <= 0 || g.num_kv_heads <= 0 || g.head_dim <= 0) return 0;
  return (size_t)g.block_size * g.num_kv_heads * g.head_dim * 2;
}

int pa_pool_create(int32_t num_pages, pa_pool_t** out) {
  if (!out || num_pages <= 0) return PA_ERR_INVALID_ARG;
  pa_pool* p = new (std::nothrow) pa_pool();
  if (!p) return PA_ERR_INVALID_ARG;
  p->refs.assign(num_pages, 0);
  p->free_list.resize(num_pages);
  // pop order: 0, 1, 2, ... (the stack top is the back)
  for (int32_t i = 0; i < num_pages; ++i) p->free_list[i] = num_pages - 1 - i;
  *out = p;
  return PA_OK;
}

void pa_pool_destroy(pa_pool_t* p) { delete p; }

int pa_pool_alloc(pa_pool_t* p, int32_t n, int32_t* ids_out) {
  if (!p || n < 0 || (n > 0 && !ids_out)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(p->mu);
  if ((size_t)n > p->free_list.size()) return PA_ERR_OUT_OF_PAGES;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = p->free_list.back();
    p->free_list.pop_back();
    p->refs[id] = 1;
    ids_out[i] = id;
  }
  return PA_OK;
}

int pa_pool_share(pa_pool_t* p, int32_t n, const int32_t* ids) {
  if (!p || n < 0 || (n > 0 && !ids)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(p->mu);
  const int32_t np = (int32_t)p->refs.size();
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= np || p->refs[ids[i]] <= 0) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) ++p->refs[ids[i]];
  return PA_OK;
}

int pa_pool_free(pa_pool_t* p, int32_t n, const int32_t* ids) {
  if (!p || n < 0 || (n > 0 && !ids)) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(p->mu);
  const int32_t np = (int32_t)p->refs.size();
  // validate first (counting repeats) so a bad call changes nothing
  std::vector<int32_t> drop;
  drop.reserve(n);
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= np) return PA_ERR_INVALID_ARG;
    drop.push_back(ids[i]);
  }
  std::sort(drop.begin(), drop.end());
  for (size_t i = 0; i < drop.size();) {
    size_t k = i;
    while (k < drop.size() && drop[k] == drop[i]) ++k;
    if ((int64_t)(k - i) > p->refs[drop[i]]) return PA_ERR_INVALID_ARG;
    i = k;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (--p->refs[ids[i]] == 0) p->free_list.push_back(ids[i]);
  }
  return PA_OK;
}

int pa_pool_cow(pa_pool_t* p, int32_t n, const int32_t* ids, int32_t* ids_out) {
  if (!p || n < 0 || (n > 0 && (!ids || !ids_out))) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(p->mu);
  const int32_t np = (int32_t)p->refs.size();
  // validate and count the copies first (entry by entry), so a failing call changes nothing
  size_t copies = 0;
  {
    std::vector<int32_t> seen_ids;
    std::vector<int32_t> seen_refs;
    for (int32_t i = 0; i < n; ++i) {
      const int32_t id = ids[i];
      if (id < 0 || id >= np || p->refs[id] <= 0) return PA_ERR_INVALID_ARG;
      size_t k = 0;
      while (k < seen_ids.size() && seen_ids[k] != id) ++k;
      if (k == seen_ids.size()) {
        seen_ids.push_back(id);
        seen_refs.push_back(p->refs[id]);
      }
      if (seen_refs[k] > 1) {
        --seen_refs[k];
        ++copies;
      }
    }
  }
  if (copies > p->free_list.size()) return PA_ERR_OUT_OF_PAGES;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (p->refs[id] > 1) {
      --p->refs[id];
      const int32_t fresh = p->free_list.back();
      p->free_list.pop_back();
      p->refs[fresh] = 1;
      ids_out[i] = fresh;
    } else {
      ids_out[i] = id;
    }
  }
  return PA_OK;
}

int32_t pa_pool_num_free(const pa_pool_t* p) {
  if (!p) return -1;
  std::lock_guard<std::mutex> lock(const_cast<pa_pool*>(p)->mu);
  return (int32_t)p->free_list.size();
}

int32_t pa_pool_refcount(const pa_pool_t* p, int32_t id) {
  if (!p) return -1;
  std::lock_guard<std::mutex> lock(const_cast<pa_pool*>(p)->mu);
  if (id < 0 || id >= (int32_t)p->refs.size()) return -1;
  return p->refs[id];
}

// ---------------------------------------------------------------------------------------
// device entry points
// ---------------------------------------------------------------------------------------
int pa_kv_append(pa_geom_t g, const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* cu_new_lens, const int32_t* ctx_lens, int32_t n_seqs,
                 int32_t n_new_tokens, void* stream) {
  int st = pa_geom_check(g);
  if (st != PA_OK) return st;
  if (n_new_tokens < 0 || n_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (n_new_tokens == 0) return PA_OK;
  if (n_seqs == 0) return PA_ERR_INVALID_ARG;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !cu_new_lens || !ctx_lens)
    return PA_ERR_INVALID_ARG;
  if ((int64_t)n_new_tokens * g.num_kv_heads > (int64_t)INT32_MAX - 4) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_kv_append(to_launch(g), k_new, v_new, k_pool, v_pool, block_tables,
                                         max_blocks_per_seq, cu_new_lens, ctx_lens, n_seqs,
                                         n_new_tokens, static_cast<hipStream_t>(stream)));
}

int pa_rope_kv_append(pa_geom_t g, const void* q, void* q_out, const void* k_new,
                      const void* v_new, void* k_pool, void* v_pool, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* cu_new_lens,
                      const int32_t* ctx_lens, int32_t n_seqs, int32_t n_new_tokens,
                      double rope_theta, const float* inv_freq, void* stream) {
  int st = pa_geom_check(g);
  if (st != PA_OK) return st;
  if (n_new_tokens < 0 || n_seqs < 0 || max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (!inv_freq && !(rope_theta > 0.0 && std::isfinite(rope_theta))) return PA_ERR_INVALID_ARG;
  if ((q == nullptr) != (q_out == nullptr)) return PA_ERR_INVALID_ARG;
  if (n_new_tokens == 0) return PA_OK;
  if (n_seqs == 0) return PA_ERR_INVALID_ARG;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !cu_new_lens || !ctx_lens)
    return PA_ERR_INVALID_ARG;
  if ((int64_t)n_new_tokens * g.num_kv_heads > (int64_t)INT32_MAX - 4) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_rope_kv_append(
      to_launch(g), q, q_out, k_new, v_new, k_pool, v_pool, block_tables, max_blocks_per_seq,
      cu_new_lens, ctx_lens, n_seqs, n_new_tokens, rope_theta, inv_freq,
      static_cast<hipStream_t>(stream)));
}

int pa_copy_pages(pa_geom_t g, void* k_pool, void* v_pool, const int32_t* src_pages,
                  const int32_t* dst_pages, int32_t n, void* stream) {
  int st = pa_geom_check(g);
  if (st != PA_OK) return st;
  if (n < 0) return PA_ERR_INVALID_ARG;
  if (n == 0) return PA_OK;
  if (!k_pool || !v_pool || !src_pages || !dst_pages) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_copy_pages(to_launch(g), k_pool, v_pool, src_pages, dst_pages, n,
                                          static_cast<hipStream_t>(stream)));
}

int pa_residual_rmsnorm(const void* x, const void* residual_in, void* residual_out,
                        const void* gamma, void* out, int32_t n_rows, int32_t hidden, float eps,
                        void* stream) {
  if (n_rows < 0 || hidden <= 0 || hidden % 8 != 0 || !(eps >= 0.f) || !std::isfinite(eps))
    return PA_ERR_INVALID_ARG;
  if (hidden > pa::rmsnorm_max_hidden()) return PA_ERR_UNSUPPORTED;
  if ((residual_in == nullptr) != (residual_out == nullptr)) return PA_ERR_INVALID_ARG;
  if (n_rows == 0) return PA_OK;
  if (!x || !gamma || !out) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_residual_rmsnorm(x, residual_in, residual_out, gamma, out, n_rows,
                                                hidden, eps, compute_units(),
                                                static_cast<hipStream_t>(stream)));
}

int pa_silu_mul(const void* gate, const void* up, int64_t ld_in, void* out, int64_t ld_out,
                int32_t n_rows, int32_t width, void* stream) {
  if (n_rows < 0 || width <= 0 || width % 8 != 0) return PA_ERR_INVALID_ARG;
  if (ld_in < width || ld_out < width || ld_in % 8 != 0 || ld_out % 8 != 0)
    return PA_ERR_INVALID_ARG;
  if (width > pa::silu_max_width()) return PA_ERR_UNSUPPORTED;
  if (n_rows == 0) return PA_OK;
  if (!gate || !up || !out) return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_silu_mul(gate, up, ld_in, out, ld_out, n_rows, width,
                                        compute_units(), static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_partition_tokens(pa_geom_t g, int32_t n_seqs, int32_t max_ctx_len,
                                   int32_t partition_tokens) {
  const int st = decode_args_ok(g, n_seqs, max_ctx_len, partition_tokens);
  if (st != PA_OK) return st;
  const pa::DecodePlan p = pa::plan_decode(n_seqs, max_ctx_len, g.num_kv_heads, partition_tokens,
                                           compute_units());
  return (int32_t)std::min<int64_t>(p.tiles_per_worker * 64, INT32_MAX);
}

size_t pa_decode_workspace_bytes(pa_geom_t g, int32_t n_seqs, int32_t max_ctx_len,
                                 int32_t partition_tokens) {
  if (decode_args_ok(g, n_seqs, max_ctx_len, partition_tokens) != PA_OK) return 0;
  return pa::plan_decode(n_seqs, max_ctx_len, g.num_kv_heads, partition_tokens, compute_units())
      .ws_bytes;
}

int pa_decode(pa_geom_t g, void* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* ctx_lens,
              int32_t n_seqs, int32_t max_ctx_len, float scale, int32_t partition_tokens,
              void* workspace, size_t workspace_bytes, void* stream) {
  const int st = decode_args_ok(g, n_seqs, max_ctx_len, partition_tokens);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_ctx_len > (int64_t)max_blocks_per_seq * g.block_size) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PA_ERR_INVALID_ARG;
  if (n_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !ctx_lens) return PA_ERR_INVALID_ARG;
  const pa::DecodePlan plan = pa::plan_decode(n_seqs, max_ctx_len, g.num_kv_heads,
                                              partition_tokens, compute_units());
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return PA_ERR_WORKSPACE;
  return hip_status(pa::launch_decode(to_launch(g), plan, out, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, ctx_lens, n_seqs, max_ctx_len, scale,
                                      workspace, static_cast<hipStream_t>(stream)));
}

int pa_decode_append(pa_geom_t g, void* out, const void* q, const void* k_new,
                     const void* v_new, void* k_pool, void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* ctx_lens, int32_t n_seqs, int32_t max_ctx_len, float scale,
                     int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const int st = decode_args_ok(g, n_seqs, max_ctx_len, partition_tokens);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_ctx_len > (int64_t)max_blocks_per_seq * g.block_size) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PA_ERR_INVALID_ARG;
  if (n_seqs == 0) return PA_OK;
  if (!out || !q || !k_new || !v_new || !k_pool || !v_pool || !block_tables || !ctx_lens)
    return PA_ERR_INVALID_ARG;
  const pa::DecodePlan plan = pa::plan_decode(n_seqs, max_ctx_len, g.num_kv_heads,
                                              partition_tokens, compute_units());
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return PA_ERR_WORKSPACE;
  return hip_status(pa::launch_decode(to_launch(g), plan, out, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, ctx_lens, n_seqs, max_ctx_len, scale,
                                      workspace, static_cast<hipStream_t>(stream), k_new, v_new));
}

int pa_decode_noalloc(pa_geom_t g, void* out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* ctx_lens, int32_t n_seqs, int32_t max_ctx_len, float scale,
                      int32_t partition_tokens, void* stream) {
  const int st = decode_args_ok(g, n_seqs, max_ctx_len, partition_tokens);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_ctx_len > (int64_t)max_blocks_per_seq * g.block_size) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PA_ERR_INVALID_ARG;
  if (n_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !ctx_lens) return PA_ERR_INVALID_ARG;
  const pa::DecodePlan plan = pa::plan_decode(n_seqs, max_ctx_len, g.num_kv_heads,
                                              partition_tokens, compute_units());
  if (plan.ws_bytes > (size_t)PA_DECODE_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    const hipError_t e = pa::decode_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(pa::launch_decode(to_launch(g), plan, out, q, k_pool, v_pool, block_tables,
                                      max_blocks_per_seq, ctx_lens, n_seqs, max_ctx_len, scale,
                                      ws, static_cast<hipStream_t>(stream)));
}

size_t pa_prefill_workspace_bytes(pa_geom_t g, int32_t n_seqs, int32_t max_q_len,
                                  int32_t max_ctx_len, int32_t kv_splits) {
  if (prefill_args_ok(g, n_seqs, max_q_len, max_ctx_len, kv_splits) != PA_OK) return 0;
  return pa::plan_prefill(n_seqs, max_q_len, max_ctx_len, g.num_kv_heads, kv_splits,
                          compute_units())
      .ws_bytes;
}

int pa_prefill(pa_geom_t g, void* out, const void* q, const void* k_pool, const void* v_pool,
               const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
               const int32_t* ctx_lens, int32_t n_seqs, int32_t max_q_len, int32_t max_ctx_len,
               float scale, int32_t causal, int32_t kv_splits, void* workspace,
               size_t workspace_bytes, void* stream) {
  const int st = prefill_args_ok(g, n_seqs, max_q_len, max_ctx_len, kv_splits);
  if (st != PA_OK) return st;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)max_ctx_len > (int64_t)max_blocks_per_seq * g.block_size) return PA_ERR_INVALID_ARG;
  if (max_q_len > max_ctx_len) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return PA_ERR_INVALID_ARG;
  if (n_seqs == 0 || max_q_len == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !cu_q_lens || !ctx_lens)
    return PA_ERR_INVALID_ARG;
  const pa::PrefillPlan plan = pa::plan_prefill(n_seqs, max_q_len, max_ctx_len, g.num_kv_heads,
                                                kv_splits, compute_units());
  if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes))
    return PA_ERR_WORKSPACE;
  return hip_status(pa::launch_prefill(to_launch(g), plan, out, q, k_pool, v_pool, block_tables,
                                       max_blocks_per_seq, cu_q_lens, ctx_lens, n_seqs, max_q_len,
                                       scale, causal, workspace,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// Slot scheduler: decides, step by step, which requests append how many tokens, and hands
// back the block tables, context lengths and cumulative new-token counts that
// pa_kv_append / pa_prefill / pa_decode take.
//
// Continuous batching as "Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎"
// (§连续批处理：吞吐与延迟的平衡) describes it: the batch is a fixed set of slots, one
// request each; a request goes waiting -> prefill -> decode -> done; a freed slot takes
// the next queued request; a prefill step runs on its own, a decode step runs every
// decoding slot; prefill and decode are kept apart so that long prompts do not stall
// the decoding of short requests.  Pages come from the shared pool only when a step
// writes into them ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §PagedAttention).
//
// Per step:
//   1. retire requests that have produced max_new tokens or were finished by the caller
//      (their pages go back to the pool, their slot is freed);
//   2. admit queued requests in order into the lowest free slots while the pool's free
//      pages, less the pages promised to admitted requests, cover the next request's
//      worst case ceil((prompt + max_new - 1) / block_size); the first that does not fit
//      stops admission (no overtaking), so a step can never run out of pages;
//   3. prefill if some slot is prefilling and either none decodes or the previous step
//      was not a prefill; else decode if some slot decodes; else idle;
//   4. prefill: prefilling slots in admission order take their remaining prompt tokens
//      until prefill_chunk tokens are given out; a completed prompt yields the first
//      generated token;
//   5. decode: each decoding slot appends one token.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <mutex>
#include <new>
#include <vector>

#include "pa.h"

namespace {

struct SchedReq {
  int64_t id;
  int32_t prompt;
  int32_t max_new;
  int32_t slot = -1;
  int32_t cached = 0;     // tokens whose K/V are in the cache
  int32_t generated = 0;  // tokens produced
  bool stop = false;      // finished by the caller
  std::vector<int32_t> pages;

  int32_t reserve(int32_t bs) const {
    return (int32_t)(((int64_t)prompt + max_new - 1 + bs - 1) / bs);
  }
  bool done() const { return stop || generated >= max_new; }
  bool prefilling() const { return cached < prompt; }
};

int32_t blocks_for(int64_t tokens, int32_t bs) { return (int32_t)((tokens + bs - 1) / bs); }

}  // namespace

struct pa_sched {
  mutable std::mutex mu;
  pa_pool_t* pool = nullptr;
  int32_t num_slots = 0, bs = 0, max_blocks = 0, chunk = 0;
  std::deque<SchedReq> queue;       // submission order
  std::vector<SchedReq> active;     // admission order
  int32_t last_kind = PA_STEP_IDLE;

  bool known(int64_t id) const {
    for (const auto& r : queue)
      if (r.id == id) return true;
    for (const auto& r : active)
      if (r.id == id) return true;
    return false;
  }
  int64_t promised() const {
    int64_t p = 0;
    for (const auto& r : active) p += r.reserve(bs) - (int32_t)r.pages.size();
    return p;
  }
};

extern "C" {

int pa_sched_create(pa_pool_t* pool, int32_t num_slots, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t prefill_chunk, pa_sched_t** out) {
  if (!pool || !out || num_slots <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
      prefill_chunk <= 0)
    return PA_ERR_INVALID_ARG;
  pa_sched* s = new (std::nothrow) pa_sched();
  if (!s) return PA_ERR_INVALID_ARG;
  s->pool = pool;
  s->num_slots = num_slots;
  s->bs = block_size;
  s->max_blocks = max_blocks_per_seq;
  s->chunk = prefill_chunk;
  *out = s;
  return PA_OK;
}

void pa_sched_destroy(pa_sched_t* s) {
  if (!s) return;
  for (auto& r : s->active)
    if (!r.pages.empty()) pa_pool_free(s->pool, (int32_t)r.pages.size(), r.pages.data());
  delete s;
}

int pa_sched_submit(pa_sched_t* s, int64_t req_id, int32_t prompt_len, int32_t max_new_tokens) {
  if (!s || prompt_len < 1 || max_new_tokens < 1) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(s->mu);
  SchedReq r;
  r.id = req_id;
  r.prompt = prompt_len;
  r.max_new = max_new_tokens;
  if (r.reserve(s->bs) > s->max_blocks) return PA_ERR_UNSUPPORTED;
  if (s->known(req_id)) return PA_ERR_INVALID_ARG;
  s->queue.push_back(std::move(r));
  return PA_OK;
}

int pa_sched_finish(pa_sched_t* s, int64_t req_id) {
  if (!s) return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(s->mu);
  for (auto it = s->queue.begin(); it != s->queue.end(); ++it) {
    if (it->id == req_id) {
      s->queue.erase(it);
      return PA_OK;
    }
  }
  for (auto& r : s->active) {
    if (r.id == req_id) {
      r.stop = true;
      return PA_OK;
    }
  }
  return PA_ERR_INVALID_ARG;
}

int32_t pa_sched_pending(const pa_sched_t* s) {
  if (!s) return -1;
  std::lock_guard<std::mutex> lock(s->mu);
  return (int32_t)(s->queue.size() + s->active.size());
}

int pa_sched_step(pa_sched_t* s, pa_sched_step_t* info, int64_t* req_ids, int32_t* slots,
                  int32_t* block_tables, int32_t* ctx_lens, int32_t* cu_new_lens,
                  int64_t* finished) {
  if (!s || !info || !req_ids || !slots || !block_tables || !ctx_lens || !cu_new_lens ||
      !finished)
    return PA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(s->mu);
  *info = pa_sched_step_t{};

  // 1. retire
  int32_t n_fin = 0;
  {
    std::vector<SchedReq> keep;
    keep.reserve(s->active.size());
    for (auto& r : s->active) {
      if (r.done()) {
        if (!r.pages.empty()) pa_pool_free(s->pool, (int32_t)r.pages.size(), r.pages.data());
        finished[n_fin++] = r.id;
      } else {
        keep.push_back(std::move(r));
      }
    }
    s->active.swap(keep);
  }
  info->n_finished = n_fin;

  // 2. admit
  while (!s->queue.empty() && (int32_t)s->active.size() < s->num_slots) {
    SchedReq& head = s->queue.front();
    const int64_t room = (int64_t)pa_pool_num_free(s->pool) - s->promised();
    if (head.reserve(s->bs) > room) break;
    std::vector<char> used(s->num_slots, 0);
    for (const auto& r : s->active) used[r.slot] = 1;
    int32_t slot = 0;
    while (used[slot]) ++slot;
    head.slot = slot;
    s->active.push_back(std::move(head));
    s->queue.pop_front();
  }

  // 3. kind
  bool any_pre = false, any_dec = false;
  for (const auto& r : s->active) (r.prefilling() ? any_pre : any_dec) = true;
  int32_t kind = PA_STEP_IDLE;
  if (any_pre && (!any_dec || s->last_kind != PA_STEP_PREFILL))
    kind = PA_STEP_PREFILL;
  else if (any_dec)
    kind = PA_STEP_DECODE;

  // 4./5. rows: first the token counts, then the pages they need (all or nothing)
  std::vector<int32_t> rows, n_new;  // indices into active, tokens appended
  if (kind == PA_STEP_PREFILL) {
    int32_t budget = s->chunk;
    for (int32_t i = 0; i < (int32_t)s->active.size() && budget > 0; ++i) {
      const SchedReq& r = s->active[i];
      if (!r.prefilling()) continue;
      const int32_t n = std::min(r.prompt - r.cached, budget);
      budget -= n;
      rows.push_back(i);
      n_new.push_back(n);
    }
  } else if (kind == PA_STEP_DECODE) {
    for (int32_t i = 0; i < (int32_t)s->active.size(); ++i) {
      if (s->active[i].prefilling()) continue;
      rows.push_back(i);
      n_new.push_back(1);
    }
  }
  int64_t need = 0;
  for (size_t k = 0; k < rows.size(); ++k) {
    const SchedReq& r = s->active[rows[k]];
    need += blocks_for((int64_t)r.cached + n_new[k], s->bs) - (int32_t)r.pages.size();
  }
  // One pool call takes every page of the step (all or nothing, also against other users of
  // the pool), in the order the rows then consume them.
  std::vector<int32_t> fresh((size_t)need);
  if (need > 0 && pa_pool_alloc(s->pool, (int32_t)need, fresh.data()) != PA_OK) {
    // only possible when pages promised to admitted requests were taken from the pool by
    // another user of it: nothing is scheduled
    s->last_kind = PA_STEP_IDLE;
    return PA_ERR_OUT_OF_PAGES;
  }

  int32_t total_new = 0, max_ctx = 0, max_new = 0;
  size_t next_page = 0;
  cu_new_lens[0] = 0;
  for (size_t k = 0; k < rows.size(); ++k) {
    SchedReq& r = s->active[rows[k]];
    const int32_t n = n_new[k];
    const int32_t grow = blocks_for((int64_t)r.cached + n, s->bs) - (int32_t)r.pages.size();
    for (int32_t i = 0; i < grow; ++i) r.pages.push_back(fresh[next_page++]);
    r.cached += n;
    if (kind == PA_STEP_PREFILL) {
      if (r.cached == r.prompt) r.generated = 1;
    } else {
      r.generated += 1;
    }
    req_ids[k] = r.id;
    slots[k] = r.slot;
    ctx_lens[k] = r.cached;
    total_new += n;
    cu_new_lens[k + 1] = total_new;
    max_ctx = std::max(max_ctx, r.cached);
    max_new = std::max(max_new, n);
    int32_t* row = block_tables + k * (size_t)s->max_blocks;
    const int32_t np = (int32_t)r.pages.size();
    std::copy(r.pages.begin(), r.pages.end(), row);
    std::fill(row + np, row + s->max_blocks, -1);
  }
  s->last_kind = kind;
  info->kind = kind;
  info->n_seqs = (int32_t)rows.size();
  info->n_new_tokens = total_new;
  info->max_ctx_len = max_ctx;
  info->max_new_len = max_new;
  return PA_OK;
}

}  // extern "C"

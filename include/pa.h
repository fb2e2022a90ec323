/*
 * pa.h -- C ABI of libpagedattn: paged KV attention for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [guide]  "tiny-vllm：从零构建高性能LLM推理引擎的完整指南"
 *   [实战]   "Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎"
 *
 * The problem, as those pages state it: the KV cache is cut into fixed-size pages
 * taken from a preallocated pool ([实战] §内存池管理); a free-page list hands pages
 * out on demand and takes them back when a request ends; pages may be shared by
 * requests with a common prefix; each sequence reaches its pages through a block table
 * ([guide] §PagedAttention); each new token's K/V is appended to the cache before it
 * attends ([guide] §推理流程：从Prefill到Decode); attention runs with online softmax
 * ([guide] §在线Softmax) on bf16 data with fp32 accumulation ([实战] §CUDA Kernel 优化,
 * 数据类型精度权衡), with grouped-query heads ([guide] §Llama 3.2 1B架构拆解).
 *
 * Conventions for every entry point:
 *   - Status: 0 (PA_OK) or a negative PA_ERR_* code.  Nothing aborts and nothing throws
 *     across the ABI.  Host-checkable errors return before anything is launched.
 *   - Device pointers are caller-owned device memory (the library never allocates or
 *     frees device memory); they must stay valid until the work queued on `stream`
 *     has finished.  `stream` is a hipStream_t passed as void* (NULL = null stream).
 *     Launches are asynchronous.
 *   - Values stored on the device (block-table entries, context lengths, cumulative
 *     lengths) are trusted, except that every kernel clamps a sequence's length to its
 *     block-table row (max_blocks_per_seq * block_size) and never dereferences a page
 *     id outside [0, num_pages): a read of such a page yields NaN in that output row,
 *     a write to it is dropped.
 *
 * Memory layout (bf16 = 2 bytes; the pages fix only a page's size, block_size x
 * head_dim x num_kv_heads values, [实战] §内存池管理; the order inside is this
 * library's choice):
 *   k_pool  [num_pages][num_kv_heads][head_dim/8][block_size][8]   bf16
 *   v_pool  [num_pages][num_kv_heads][head_dim][block_size]        bf16
 *   block_tables  int32 [n_seqs][max_blocks_per_seq]: logical block b of sequence s
 *                 lives in physical page block_tables[s*max_blocks_per_seq + b]
 *   q, out, k_new, v_new: token-major rows [tokens][heads][head_dim] bf16
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * One pool pair holds one layer; other layers are served by calling again with their
 * pool pointers (one block table may serve all layers).
 *
 * Supported geometry: head_dim 64, block_size 16 or 32, num_q_heads = 4 * num_kv_heads
 * (the Llama-3.2-1B shape is 32 query heads over 8 KV heads).  Anything else returns
 * PA_ERR_UNSUPPORTED.
 */
#ifndef PAGEDATTN_PA_H
#define PAGEDATTN_PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,  /* null pointer, negative size, inconsistent sizes, bad page id */
  PA_ERR_OUT_OF_PAGES = -2, /* pool cannot satisfy an allocation */
  PA_ERR_UNSUPPORTED = -3,  /* geometry outside the supported set */
  PA_ERR_WORKSPACE = -4,    /* split-K workspace missing or too small */
  PA_ERR_HIP = -5           /* a HIP runtime call or launch failed; see pa_last_hip_error */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* pa_status_string(int status);

/* The hipError_t value behind the calling thread's most recent PA_ERR_HIP. */
int pa_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int pa_version(void);

typedef struct pa_geom {
  int32_t num_pages;    /* physical pages in each pool */
  int32_t block_size;   /* tokens per page: 16 or 32 */
  int32_t num_q_heads;  /* query heads */
  int32_t num_kv_heads; /* KV heads */
  int32_t head_dim;     /* 64 */
} pa_geom_t;

/* PA_OK if `g` is supported, else PA_ERR_UNSUPPORTED (or PA_ERR_INVALID_ARG for
 * non-positive fields). */
int pa_geom_check(pa_geom_t g);

/* Bytes of one page of one pool (K or V) of one layer:
 * block_size * num_kv_heads * head_dim * 2.  16384 for 16 tokens at 8 x 64 ([实战]
 * §内存池管理).  0 if a field is non-positive. */
size_t pa_page_bytes(pa_geom_t g);

/* ---------------------------------------------------------------------------------
 * Host page pool: the free-page list of [实战] §内存池管理, with a reference count per
 * page so prefix pages can be shared (same section: different requests may share
 * pages).  It owns host metadata only -- no device memory.  Calls on one pool are
 * serialised internally (thread-safe).
 * ------------------------------------------------------------------------------- */
typedef struct pa_pool pa_pool_t;

/* Create a pool of `num_pages` free pages (ids 0..num_pages-1).  *out receives the
 * handle.  PA_ERR_INVALID_ARG if num_pages <= 0 or out is NULL. */
int pa_pool_create(int32_t num_pages, pa_pool_t** out);

/* Destroy a pool (NULL is ignored). */
void pa_pool_destroy(pa_pool_t* p);

/* Take `n` pages off the free list into ids_out[0..n-1], each with reference count 1.
 * The free list is a stack: a fresh pool hands out 0, 1, 2, ... in that order, and a
 * page that returns to it is the next one handed out.
 * All or nothing: PA_ERR_OUT_OF_PAGES leaves the pool unchanged. */
int pa_pool_alloc(pa_pool_t* p, int32_t n, int32_t* ids_out);

/* Add one reference to each of the `n` allocated pages in `ids` (a prefix shared by
 * one more sequence).  PA_ERR_INVALID_ARG (and no change) if any id is out of range
 * or free. */
int pa_pool_share(pa_pool_t* p, int32_t n, const int32_t* ids);

/* Drop one reference from each page in `ids`; a page whose count reaches 0 returns to
 * the free list.  PA_ERR_INVALID_ARG (and no change) if any id is out of range or
 * already free, counting repeats within `ids`. */
int pa_pool_free(pa_pool_t* p, int32_t n, const int32_t* ids);

/* Copy-on-write decision ([guide] §PagedAttention: shared pages make copy-on-write
 * straightforward).  `ids` are the pages a caller is about to write (its block-table
 * entries), taken in order: an entry whose page has more than one reference at its turn
 * drops one reference and receives a fresh page (reference count 1) in ids_out[i]; an
 * entry whose page has a single reference keeps it (ids_out[i] = ids[i]).  The caller then
 * copies every changed pair with pa_copy_pages and points its block table at ids_out.
 * All or nothing: PA_ERR_OUT_OF_PAGES (not enough free pages for the copies) or
 * PA_ERR_INVALID_ARG (an id out of range or free) leaves the pool unchanged. */
int pa_pool_cow(pa_pool_t* p, int32_t n, const int32_t* ids, int32_t* ids_out);

/* Pages currently on the free list (-1 for a NULL pool). */
int32_t pa_pool_num_free(const pa_pool_t* p);

/* Reference count of page `id` (0 = free; -1 for a bad pool or id). */
int32_t pa_pool_refcount(const pa_pool_t* p, int32_t id);

/* ---------------------------------------------------------------------------------
 * kv_append ([guide] §推理流程：从Prefill到Decode: a token's K/V goes into the cache
 * before the token attends).  Copies n_new_tokens rows of k_new/v_new into the pools,
 * bit for bit.  Rows are packed by sequence: rows cu_new_lens[s] .. cu_new_lens[s+1]-1
 * belong to sequence s, whose length after the append is ctx_lens[s]; row j of that
 * range lands at position ctx_lens[s] - n_s + j, i.e. in page
 * block_tables[s][pos / block_size], slot pos % block_size.
 *   k_new, v_new   [n_new_tokens][num_kv_heads][head_dim] bf16 (device)
 *   k_pool, v_pool pools (device, written in place)
 *   cu_new_lens    int32 [n_seqs+1] (device), cu_new_lens[0] = 0,
 *                  cu_new_lens[n_seqs] = n_new_tokens
 *   ctx_lens       int32 [n_seqs] (device), lengths after the append
 * No two rows of one call may target the same slot.  n_new_tokens == 0 is a no-op.
 * PA_ERR_INVALID_ARG for a missing pointer, n_seqs == 0 with rows to append, or
 * n_new_tokens * num_kv_heads above 2^31 - 5.
 * ------------------------------------------------------------------------------- */
int pa_kv_append(pa_geom_t g, const void* k_new, const void* v_new, void* k_pool,
                 void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* cu_new_lens, const int32_t* ctx_lens, int32_t n_seqs,
                 int32_t n_new_tokens, void* stream);

/* ---------------------------------------------------------------------------------
 * copy_pages (the copy half of copy-on-write, [guide] §PagedAttention).  Copies whole
 * page src_pages[i] onto page dst_pages[i] in both pools (every KV head, every slot), bit
 * for bit, for i < n.
 *   src_pages, dst_pages  int32 [n] (device)
 * Pairs with an id outside [0, num_pages) or with src == dst are skipped.  The
 * destination pages must be distinct and none of them a source (the pairs run in no
 * particular order).  n == 0 is a no-op.
 * ------------------------------------------------------------------------------- */
int pa_copy_pages(pa_geom_t g, void* k_pool, void* v_pool, const int32_t* src_pages,
                  const int32_t* dst_pages, int32_t n, void* stream);

/* ---------------------------------------------------------------------------------
 * residual_rmsnorm ([guide] §Llama 3.2 1B架构拆解: RMS normalisation and a residual
 * connection around every sub-layer; [实战] §算子融合: the residual add fused into the
 * normalisation).  Per row of `hidden` values:
 *   h = x + residual_in (rounded to bf16 and stored in residual_out, the next residual),
 *   out = h / sqrt(mean(h^2) + eps) * gamma, rounded once to bf16 (nearest even).
 * Sums and products run in fp32.
 *   x, out                  [n_rows][hidden] bf16 (device)
 *   residual_in, residual_out  [n_rows][hidden] bf16 (device); residual_out may be
 *                           residual_in (in place); both NULL for h = x
 *   gamma                   [hidden] bf16 (device)
 *   hidden                  a multiple of 8, at most 8192 (else PA_ERR_UNSUPPORTED)
 *   eps                     >= 0, finite (1e-5 for the Llama 3 family)
 * PA_ERR_INVALID_ARG for a missing pointer, exactly one residual pointer, or bad sizes.
 * ------------------------------------------------------------------------------- */
int pa_residual_rmsnorm(const void* x, const void* residual_in, void* residual_out,
                        const void* gamma, void* out, int32_t n_rows, int32_t hidden, float eps,
                        void* stream);

/* ---------------------------------------------------------------------------------
 * silu_mul ([guide] §Llama 3.2 1B架构拆解: SiLU of the gate projection times the up
 * projection, element-wise).  out[t][j] = g / (1 + e^-g) * u with g = gate[t*ld_in + j],
 * u = up[t*ld_in + j], in fp32, rounded once to bf16; written to out[t*ld_out + j], for
 * j < width.  A concatenated [n_rows][2*width] gate|up buffer is gate = base,
 * up = base + width, ld_in = 2*width.
 *   width, ld_in, ld_out    multiples of 8 with ld_in, ld_out >= width (elements);
 *                           width at most 2^24 (else PA_ERR_UNSUPPORTED)
 * PA_ERR_INVALID_ARG for a missing pointer or bad sizes.
 * ------------------------------------------------------------------------------- */
int pa_silu_mul(const void* gate, const void* up, int64_t ld_in, void* out, int64_t ld_out,
                int32_t n_rows, int32_t width, void* stream);

/* ---------------------------------------------------------------------------------
 * rope_kv_append ([guide] §Llama 3.2 1B架构拆解: rotary position encoding turns Q and K
 * by the token's position before attention; §推理流程：从Prefill到Decode: K/V join the
 * cache before the token attends).  For the same rows, positions and pages as
 * pa_kv_append: K is rotated and appended, V is appended unchanged, and Q (when given)
 * is rotated into q_out.  Pair i of a head vector is (x[i], x[i + head_dim/2]) and turns
 * counter-clockwise by pos * f_i:  (a, b) -> (a cos t - b sin t, b cos t + a sin t),
 * with f_i = rope_theta^(-2i/head_dim), or f_i = inv_freq[i] when inv_freq is given
 * (any rescaled frequency table).  Angles are formed and reduced in fp64, the rotation
 * runs in fp32 and each result is rounded once to bf16 (nearest even).
 *   q, q_out        [n_new_tokens][num_q_heads][head_dim] bf16 (device); q_out may be
 *                   q (in place); both NULL to rotate K only
 *   k_new, v_new, block_tables, cu_new_lens, ctx_lens, n_seqs, n_new_tokens: as for
 *                   pa_kv_append (positions ctx_lens[s] - n_s + j)
 *   rope_theta      base of the frequency table (> 0, finite; 500000 for the Llama 3
 *                   family); ignored when inv_freq is given
 *   inv_freq        NULL or head_dim/2 fp32 frequencies (device)
 * A row whose position falls outside its block-table row, or whose page id is out of
 * range, is not appended (its Q is still rotated).  PA_ERR_INVALID_ARG for a missing
 * pointer, exactly one of q / q_out NULL, a bad rope_theta without inv_freq, or sizes
 * as for pa_kv_append.
 * ------------------------------------------------------------------------------- */
int pa_rope_kv_append(pa_geom_t g, const void* q, void* q_out, const void* k_new,
                      const void* v_new, void* k_pool, void* v_pool,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* cu_new_lens, const int32_t* ctx_lens, int32_t n_seqs,
                      int32_t n_new_tokens, double rope_theta, const float* inv_freq,
                      void* stream);

/* ---------------------------------------------------------------------------------
 * Decode ([guide] §推理流程, §在线Softmax): one query row per sequence, the newest
 * token at position ctx_lens[s]-1, attending to all ctx_lens[s] keys (so the token's
 * own K/V must already be appended).  Every (sequence, KV head) pair is streamed once
 * for all query heads of its group with a running max and running sum per head.
 * The work is cut over "workers": the (sequence, KV head) pairs, each a run of
 * ceil(ctx/64) tiles of 64 tokens, are laid end to end and every worker takes a
 * contiguous share: 27 parts for the four waves of an even-numbered workgroup, 25 for
 * those of an odd one, since the odd-numbered XCDs stream the loads more slowly, with
 * the stream measured in units of two per tile and one per pair (a pair's end costs
 * about half a tile); with fewer than two tiles per worker, equal shares of tiles.  A pair may be split between
 * workers; each worker then leaves an fp32 partial (max, sum, unnormalised output) in
 * `workspace` and a second kernel merges the partials of split pairs by log-sum-exp in a
 * fixed order.  The cut depends only on the tile count and the worker count.
 *   out, q          [n_seqs][num_q_heads][head_dim] bf16 (device)
 *   ctx_lens        int32 [n_seqs] (device); 0 gives a zero row; values above
 *                   max_ctx_len are treated as max_ctx_len
 *   max_ctx_len     host upper bound of ctx_lens (0 <= max_ctx_len <=
 *                   max_blocks_per_seq * block_size); with n_seqs it bounds the work
 *                   (n_seqs * num_kv_heads * ceil(max_ctx_len/64) < 2^31)
 *   scale           multiplies q.k before the softmax: finite and > 0
 *                   (1/sqrt(head_dim) = 0.125); anything else gives PA_ERR_INVALID_ARG
 *   partition_tokens  0: four workers per compute unit of the current device (more if
 *                   a share would exceed 56 * num_kv_heads tiles); else a positive
 *                   multiple of 64, and enough workers that none streams more than that
 *                   many tokens (nor more than 56 * num_kv_heads tiles).  Other values
 *                   give PA_ERR_INVALID_ARG.
 *   workspace       device scratch of at least pa_decode_workspace_bytes(...) bytes
 *                   for the same arguments (on the same device); may be NULL when that
 *                   size is 0.  With W workers it is 2W * 4 * (64 * 4 + 8) + 8 * (W + 1)
 *                   bytes (two fp32 partial slots per worker, then W + 1 int32 pairs), or
 *                   0 when no pair can be split (ceil(max_ctx_len/64) <= 1 or W = 1).  Its contents need no initialisation and are scratch
 *                   after the call; concurrent calls need separate workspaces.
 * pa_decode_partition_tokens returns the most tokens one worker streams for these
 * arguments (a multiple of 64), or a negative status.
 * ------------------------------------------------------------------------------- */
int32_t pa_decode_partition_tokens(pa_geom_t g, int32_t n_seqs, int32_t max_ctx_len,
                                   int32_t partition_tokens);
size_t pa_decode_workspace_bytes(pa_geom_t g, int32_t n_seqs, int32_t max_ctx_len,
                                 int32_t partition_tokens);
int pa_decode(pa_geom_t g, void* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* ctx_lens,
              int32_t n_seqs, int32_t max_ctx_len, float scale, int32_t partition_tokens,
              void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * decode_append: the decode step's append and attention in one launch ([guide]
 * §推理流程：从Prefill到Decode: each decode step appends one token's K/V, then attends).
 * Row s of k_new / v_new ([n_seqs][num_kv_heads][head_dim] bf16, device) is the K/V of
 * position ctx_lens[s] - 1 of sequence s (ctx_lens counts it, as for pa_decode).  It is
 * written into the pools at that position, exactly as pa_kv_append with one row per
 * sequence would write it (not written if the page id is out of range; nothing for
 * ctx_lens[s] = 0), and the query attends over all ctx_lens[s] tokens, the new one
 * included.  Outputs and pools equal, bit for bit, those of pa_kv_append
 * (cu_new_lens = 0, 1, ..., n_seqs) followed by pa_decode with the same arguments.
 * Every other argument, the workspace and the errors are as for pa_decode; k_pool /
 * v_pool are written.  ctx_lens[s] must not exceed max_ctx_len (nor max_blocks_per_seq *
 * block_size): a sequence past that bound is not clamped as pa_decode clamps it, since
 * its new token would land on a cached one; nothing is written for it and its output
 * row is NaN.
 * ------------------------------------------------------------------------------- */
int pa_decode_append(pa_geom_t g, void* out, const void* q, const void* k_new,
                     const void* v_new, void* k_pool, void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* ctx_lens, int32_t n_seqs, int32_t max_ctx_len, float scale,
                     int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * decode_noalloc: pa_decode for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments,
 * outputs and errors are those of pa_decode without the workspace: the split-K partials
 * go to a device array of the library's own, PA_DECODE_SCRATCH_BYTES per device, held
 * until the process ends.  The call allocates and frees nothing.  It returns
 * PA_ERR_WORKSPACE, before any launch, when pa_decode_workspace_bytes(...) for the same
 * arguments exceeds PA_DECODE_SCRATCH_BYTES, i.e. with more than 7935 workers (the
 * automatic partition uses four per compute unit, 1024 on MI355X, unless a batch needs
 * more; a small explicit partition_tokens can ask for more).  The scratch needs no
 * initialisation.  Every
 * call on one device shares that device's array: calls that overlap in time on one
 * device (other streams, other threads) race on it and must be serialised by the caller.
 * ------------------------------------------------------------------------------- */
#define PA_DECODE_SCRATCH_BYTES (16u << 20)
int pa_decode_noalloc(pa_geom_t g, void* out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* ctx_lens, int32_t n_seqs, int32_t max_ctx_len, float scale,
                      int32_t partition_tokens, void* stream);

/* ---------------------------------------------------------------------------------
 * Prefill, whole prompts or chunks ([guide] §推理流程: prefill handles every prompt
 * token in parallel; [实战] §算子融合: tiled attention with online softmax never
 * materialises the seq x seq score matrix).  Query rows are packed by sequence: rows
 * cu_q_lens[s] .. cu_q_lens[s+1]-1 belong to sequence s; row i of it sits at position
 * ctx_lens[s] - q_len_s + i and sees keys 0..position (causal != 0) or all
 * ctx_lens[s] keys (causal == 0).  Keys before the chunk come from earlier appends,
 * so a chunk attends to the cached prefix.  Matrix products run on bf16 MFMA with fp32
 * accumulation.  One workgroup per (tile of 32 query rows, sequence, KV head).  When the
 * call has fewer tiles than compute units, a workgroup runs two groups of four waves that
 * take alternate 64-key stages of its tile and merge their results in LDS; with at most
 * half as many tiles as compute units, two workgroups share each tile, two query heads
 * each, and run four key groups that take every fourth stage.  When the grid is still
 * small, each tile's keys are also split into pieces whose fp32 partials (max, sum,
 * unnormalised output) a second kernel merges by log-sum-exp in piece order.
 *   out, q      [n_q_tokens][num_q_heads][head_dim] bf16 (device),
 *               n_q_tokens = cu_q_lens[n_seqs]
 *   cu_q_lens   int32 [n_seqs+1] (device); q_len_s <= ctx_lens[s] required
 *   max_q_len   host upper bound of q_len_s (sizes the grid: rows past it are not written)
 *   max_ctx_len host upper bound of ctx_lens (<= max_blocks_per_seq * block_size)
 *   scale       as for pa_decode: finite and > 0
 *   kv_splits   0: automatic, from the T tiles below and the C compute units of the
 *               current device, with W = T workgroups per piece (W = 2 T when 2 T <= C):
 *               with T >= C, enough pieces for 2 C workgroups; with T < C (key groups),
 *               enough for C / 2 workgroups; 1 when W already reaches that, and always
 *               at most 8 and at most ceil(max_ctx_len/64).  Else that many pieces,
 *               1 .. 8.  Other values give PA_ERR_INVALID_ARG.
 *   workspace   device scratch of at least pa_prefill_workspace_bytes(...) bytes for the
 *               same arguments (on the same device); may be NULL when that size is 0.
 *               With T = ceil(max_q_len/32) * n_seqs * num_kv_heads tiles and P pieces
 *               it is T * P * 4 * 32 * (64 * 4 + 8) bytes, or 0 when P = 1.  Its
 *               contents need no initialisation and are scratch after the call;
 *               concurrent calls need separate workspaces.
 * ceil(max_q_len/32) * n_seqs * num_kv_heads * 8 must stay below 2^31.
 * ------------------------------------------------------------------------------- */
size_t pa_prefill_workspace_bytes(pa_geom_t g, int32_t n_seqs, int32_t max_q_len,
                                  int32_t max_ctx_len, int32_t kv_splits);
int pa_prefill(pa_geom_t g, void* out, const void* q, const void* k_pool, const void* v_pool,
               const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* cu_q_lens, const int32_t* ctx_lens, int32_t n_seqs,
               int32_t max_q_len, int32_t max_ctx_len, float scale, int32_t causal,
               int32_t kv_splits, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Slot scheduler: continuous batching as [实战] §连续批处理：吞吐与延迟的平衡 describes it.
 * The batch is a fixed set of `num_slots` slots, one request each; a request goes
 * waiting -> prefill -> decode -> done; a freed slot takes the next queued request; a
 * prefill step runs on its own, a decode step runs every decoding slot, and the two
 * alternate while both have work, so a long prompt cannot stall decoding.  Pages come
 * from `pool` only when a step first writes into them ([guide] §PagedAttention).
 * Host only: it launches nothing and touches no device memory.  Calls on one scheduler
 * are serialised internally.
 *
 * pa_sched_step, in order:
 *   1. retires every request that has produced max_new_tokens tokens or was passed to
 *      pa_sched_finish: its pages go back to the pool, its id is written to finished[];
 *   2. admits queued requests, oldest first, into the lowest free slots while the pool's
 *      free pages, less the pages still promised to admitted requests, cover the next
 *      request's worst case ceil((prompt_len + max_new_tokens - 1) / block_size); the
 *      first request that does not fit stops admission (no overtaking);
 *   3. chooses the kind: PA_STEP_PREFILL if some slot is prefilling and either none is
 *      decoding or the previous step was not a prefill step; else PA_STEP_DECODE if some
 *      slot is decoding; else PA_STEP_IDLE;
 *   4. prefill: prefilling slots in admission order take their remaining prompt tokens
 *      until prefill_chunk tokens are given out; a slot whose prompt completes has
 *      produced its first token and decodes from the next step on;
 *   5. decode: every decoding slot appends one token (its latest) and produces the next.
 * Row k of the step (k < n_seqs, admission order) is request req_ids[k] in slot
 * slots[k]; it appends rows cu_new_lens[k] .. cu_new_lens[k+1]-1 at positions
 * ctx_lens[k] - n_k .. ctx_lens[k] - 1 and then attends over ctx_lens[k] tokens through
 * block_tables[k][0 .. ceil(ctx_lens[k]/block_size) - 1] (entries past that are -1).
 * These are the arguments of pa_kv_append / pa_rope_kv_append, then pa_prefill
 * (cu_q_lens = cu_new_lens, max_q_len = info->max_new_len) or pa_decode, once copied to
 * the device.  A request produces its tokens over one prefill pass of prompt_len tokens
 * and max_new_tokens - 1 decode steps; the token values belong to the caller.
 * ------------------------------------------------------------------------------- */
typedef struct pa_sched pa_sched_t;

enum { PA_STEP_IDLE = 0, PA_STEP_PREFILL = 1, PA_STEP_DECODE = 2 };

typedef struct pa_sched_step {
  int32_t kind;         /* PA_STEP_* */
  int32_t n_seqs;       /* rows in this step */
  int32_t n_new_tokens; /* cu_new_lens[n_seqs] */
  int32_t max_ctx_len;  /* largest ctx_lens[k] */
  int32_t max_new_len;  /* largest n_k (max_q_len for pa_prefill) */
  int32_t n_finished;   /* ids written to finished[] */
} pa_sched_step_t;

/* Create a scheduler over `pool`, which must outlive it (other users may share the pool:
 * admission counts its free pages at every step).  num_slots, block_size (tokens per
 * page), max_blocks_per_seq (the length of a block-table row) and prefill_chunk (prompt
 * tokens per prefill step) must be >= 1, else PA_ERR_INVALID_ARG. */
int pa_sched_create(pa_pool_t* pool, int32_t num_slots, int32_t block_size,
                    int32_t max_blocks_per_seq, int32_t prefill_chunk, pa_sched_t** out);

/* Destroy a scheduler; pages held by its requests go back to the pool (NULL ignored). */
void pa_sched_destroy(pa_sched_t* s);

/* Queue a request.  PA_ERR_INVALID_ARG for prompt_len < 1, max_new_tokens < 1 or an id
 * already queued or active; PA_ERR_UNSUPPORTED when its worst case needs more than
 * max_blocks_per_seq pages (it could never run).  Nothing changes on error. */
int pa_sched_submit(pa_sched_t* s, int64_t req_id, int32_t prompt_len, int32_t max_new_tokens);

/* Stop a request early (say, at an end-of-sequence token): a queued one leaves the queue
 * at once; an active one is retired by the next step.  PA_ERR_INVALID_ARG if unknown. */
int pa_sched_finish(pa_sched_t* s, int64_t req_id);

/* Requests queued or active (-1 for NULL). */
int32_t pa_sched_pending(const pa_sched_t* s);

/* Decide and record the next step (see above).  Caller-owned host arrays, capacities:
 * req_ids, slots, ctx_lens, finished: num_slots; cu_new_lens: num_slots + 1;
 * block_tables: num_slots * max_blocks_per_seq.  PA_ERR_INVALID_ARG for a NULL pointer.
 * PA_ERR_OUT_OF_PAGES only when another user of the pool took pages promised to admitted
 * requests: then the retirements and admissions of the call stand (finished[] and
 * info->n_finished are filled), no tokens are scheduled and info->kind is PA_STEP_IDLE. */
int pa_sched_step(pa_sched_t* s, pa_sched_step_t* info, int64_t* req_ids, int32_t* slots,
                  int32_t* block_tables, int32_t* ctx_lens, int32_t* cu_new_lens,
                  int64_t* finished);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_PA_H */

// Internal launchers behind the C ABI (include/pa.h).  Arguments are validated by the
// ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kHeadDim = 64;  // head_dim the kernels are built for
constexpr int kGroup = 4;     // query heads per KV head

struct LaunchGeom {
  int num_pages;
  int block_size;    // 16 or 32
  int num_q_heads;   // 4 * num_kv_heads
  int num_kv_heads;
};

hipError_t launch_kv_append(const LaunchGeom& geo, const void* k_new, const void* v_new,
                            void* k_pool, void* v_pool, const int32_t* block_tables,
                            int max_blocks, const int32_t* cu_new_lens, const int32_t* ctx_lens,
                            int n_seqs, int n_new_tokens, hipStream_t stream);

// Rotary position encoding of the new Q and K rows, K appended rotated and V as is.
// inv_freq: head_dim/2 frequencies (device) or nullptr for rope_theta^(-2i/head_dim).
hipError_t launch_rope_kv_append(const LaunchGeom& geo, const void* q_in, void* q_out,
                                 const void* k_new, const void* v_new, void* k_pool,
                                 void* v_pool, const int32_t* block_tables, int max_blocks,
                                 const int32_t* cu_new_lens, const int32_t* ctx_lens,
                                 int n_seqs, int n_new_tokens, double rope_theta,
                                 const float* inv_freq, hipStream_t stream);

// Copy whole pages src_pages[i] -> dst_pages[i] (device id arrays) in both pools.
hipError_t launch_copy_pages(const LaunchGeom& geo, void* k_pool, void* v_pool,
                             const int32_t* src_pages, const int32_t* dst_pages, int n,
                             hipStream_t stream);

// Residual add + RMS normalisation of bf16 rows, and the SiLU-gated product.
int rmsnorm_max_hidden();
// Widest row pa_silu_mul takes: the column groups of a row go on grid axis y.
int silu_max_width();
hipError_t launch_residual_rmsnorm(const void* x, const void* residual_in, void* residual_out,
                                   const void* gamma, void* out, int n_rows, int hidden,
                                   float eps, int compute_units, hipStream_t stream);
hipError_t launch_silu_mul(const void* gate, const void* up, int64_t ld_in, void* out,
                           int64_t ld_out, int n_rows, int width, int compute_units,
                           hipStream_t stream);

// Decode: workgroups of four waves; every wave is one stream-K worker.  A wave of an
// even-numbered workgroup takes kWeightEven parts of the tile stream, one of an odd one
// kWeightOdd (odd XCDs stream the decode loads more slowly).
constexpr int kDecodeWaves = 4;
constexpr int64_t kWeightEven = 27;
constexpr int64_t kWeightOdd = 25;
// A worker's range is at most this many tiles per KV head (so it touches at most this
// many sequences plus two, which its lanes can hold).
constexpr int kDecodeMaxSeqsPerRange = 56;
// Sequences whose context lengths a decode workgroup keeps in LDS (beyond, it re-reads them).
constexpr int kDecodeCtxCache = 4096;

// How a decode call is cut into workers; identical on the sizing and the launch side.
struct DecodePlan {
  int64_t n_max_tiles;       // upper bound of the tile stream: n_seqs * Hkv * ceil(max_ctx/64)
  int64_t workers;           // worker waves
  int64_t tiles_per_worker;  // ceil(n_max_tiles / workers)
  bool merge;                // a segment may be cut between workers (partials + merge)
  size_t ws_bytes;           // workspace needed (0 without merge)
};

// partition_tokens 0: 4 workers per compute unit; else enough workers that none streams
// more than partition_tokens tokens (a multiple of 64).
DecodePlan plan_decode(int n_seqs, int max_ctx_len, int num_kv_heads, int partition_tokens,
                       int compute_units);

// Device address of the library's own split-K scratch (PA_DECODE_SCRATCH_BYTES) on the
// current device, looked up once per device.
hipError_t decode_scratch(void** ptr);

hipError_t launch_decode(const LaunchGeom& geo, const DecodePlan& plan, void* out, const void* q,
                         const void* k_pool, const void* v_pool, const int32_t* block_tables,
                         int max_blocks, const int32_t* ctx_lens, int n_seqs, int max_ctx_len,
                         float scale, void* workspace, hipStream_t stream,
                         const void* k_new = nullptr, const void* v_new = nullptr);

// Prefill: one workgroup per (query tile of 32, sequence, KV head).  With fewer tiles than
// compute units a workgroup holds two key groups of four waves that take alternate key
// stages of its tile and merge in LDS; with still too few workgroups (or fewer than two
// per compute unit) the tile's keys are also split into up to kPrefillMaxSplit pieces
// whose fp32 partials a merge kernel combines.
constexpr int kPrefillMaxSplit = 8;

struct PrefillPlan {
  int64_t items;    // tiles x sequences x KV heads (the tile grid, ceil(max_q/32) tiles each)
  int split;        // key pieces per tile (1: no merge)
  int groups;       // key groups per workgroup (1, 2 or 4)
  int heads;        // query heads per key group (4, or 2 with four key groups)
  size_t ws_bytes;  // partials (0 when split is 1)
};

// kv_splits 0: automatic; else that many pieces (1 .. kPrefillMaxSplit).
PrefillPlan plan_prefill(int n_seqs, int max_q_len, int max_ctx_len, int num_kv_heads,
                         int kv_splits, int compute_units);

hipError_t launch_prefill(const LaunchGeom& geo, const PrefillPlan& plan, void* out, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          int max_blocks, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                          int n_seqs, int max_q_len, float scale, int causal, void* workspace,
                          hipStream_t stream);

}  // namespace pa

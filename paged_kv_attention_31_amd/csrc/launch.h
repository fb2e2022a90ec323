// Internal launchers behind the C ABI (include/pa.h).  Arguments are validated by the
// ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

constexpr int kHeadDim = 64;  // head_dim the kernels are built for
constexpr int kGroup = 4;     // query heads per KV head

struct LaunchGeom {
  int num_pages;
  int block_size;    // 16 or 32
  int num_q_heads;   // 4 * num_kv_heads
  int num_kv_heads;
};

// Decode: tokens per KV partition are a multiple of this (one tile per wave, four waves).
constexpr int kDecodeTile = 64;
constexpr int kDecodeWaves = 4;
constexpr int kDecodePartQuantum = kDecodeTile * kDecodeWaves;  // 256

hipError_t launch_kv_append(const LaunchGeom& geo, const void* k_new, const void* v_new,
                            void* k_pool, void* v_pool, const int32_t* block_tables,
                            int max_blocks, const int32_t* cu_new_lens, const int32_t* ctx_lens,
                            int n_seqs, int n_new_tokens, hipStream_t stream);

// n_parts == 1: writes bf16 `out` directly and ignores the workspace.
// n_parts  > 1: partition kernel writes fp32 partials to the workspace, merge kernel
//               writes `out`.  Workspace: o [n_seqs][n_parts][Hq][64] fp32 followed by
//               (m, l) [n_seqs][n_parts][Hq] float2.
hipError_t launch_decode(const LaunchGeom& geo, void* out, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables, int max_blocks,
                         const int32_t* ctx_lens, int n_seqs, int n_parts, int part_tokens,
                         float scale, void* workspace, hipStream_t stream);

size_t decode_workspace_bytes(int n_seqs, int n_parts, int num_q_heads);

hipError_t launch_prefill(const LaunchGeom& geo, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables, int max_blocks,
                          const int32_t* cu_q_lens, const int32_t* ctx_lens, int n_seqs,
                          int max_q_len, float scale, int causal, hipStream_t stream);

}  // namespace pa

// kv_append: write new tokens' K and V rows into their pages (a bit copy).
//
// A decoded token's K/V joins the cache before the token attends, and a prompt's K/V is
// written during prefill ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南",
// §推理流程：从Prefill到Decode).  Page and slot come from the block table
// (same page, §PagedAttention：从操作系统借来的智慧).
//
// One workgroup of 256 threads copies 4 (token, KV head) rows.  Each row is 64 bf16 of K
// and 64 of V:
//   K page layout [Hkv][8][bs][8]: 8 threads write the row's eight 16-byte pieces;
//   V page layout [Hkv][64][bs]:   64 threads write one bf16 each (row d of the page).
// The work is bandwidth-trivial next to attention (2 KB per token per layer), so the
// kernel favours simple, fully checked addressing over write coalescing.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

// sequence s with cu[s] <= t < cu[s+1] (cu ascending, cu[0] = 0)
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int n_seqs, int t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int BS>
__global__ __launch_bounds__(256) void kv_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ cu_new_lens, const int32_t* __restrict__ ctx_lens,
    int n_seqs, int n_rows, int num_kv_heads, int num_pages) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, head) row
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int tok = row / num_kv_heads;
  const int g = row - tok * num_kv_heads;
  const int s = find_seq(cu_new_lens, n_seqs, tok);
  const int first = cu_new_lens[s];
  const int n_s = cu_new_lens[s + 1] - first;
  const int pos = ctx_lens[s] - n_s + (tok - first);
  if (pos < 0 || pos >= max_blocks * BS) return;  // inconsistent lengths: drop
  const int page = block_tables[(size_t)s * max_blocks + pos / BS];
  if ((unsigned)page >= (unsigned)num_pages) return;  // bad page id: drop
  const int slot = pos % BS;
  const size_t head_base = ((size_t)page * num_kv_heads + g) * (kHeadDim * BS);
  const size_t src = (size_t)row * kHeadDim;
  if (lane < 8) {
    const uint4 piece = *reinterpret_cast<const uint4*>(k_new + src + lane * 8);
    *reinterpret_cast<uint4*>(k_pool + head_base + ((size_t)lane * BS + slot) * 8) = piece;
  }
  v_pool[head_base + (size_t)lane * BS + slot] = v_new[src + lane];
}

}  // namespace

hipError_t launch_kv_append(const LaunchGeom& geo, const void* k_new, const void* v_new,
                            void* k_pool, void* v_pool, const int32_t* block_tables,
                            int max_blocks, const int32_t* cu_new_lens, const int32_t* ctx_lens,
                            int n_seqs, int n_new_tokens, hipStream_t stream) {
  const int n_rows = n_new_tokens * geo.num_kv_heads;
  const dim3 grid((n_rows + 3) / 4);
  const dim3 block(256);
  auto* kn = static_cast<const uint16_t*>(k_new);
  auto* vn = static_cast<const uint16_t*>(v_new);
  auto* kp = static_cast<uint16_t*>(k_pool);
  auto* vp = static_cast<uint16_t*>(v_pool);
  if (geo.block_size == 16) {
    hipLaunchKernelGGL(kv_append_kernel<16>, grid, block, 0, stream, kn, vn, kp, vp, block_tables,
                       max_blocks, cu_new_lens, ctx_lens, n_seqs, n_rows, geo.num_kv_heads,
                       geo.num_pages);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<32>, grid, block, 0, stream, kn, vn, kp, vp, block_tables,
                       max_blocks, cu_new_lens, ctx_lens, n_seqs, n_rows, geo.num_kv_heads,
                       geo.num_pages);
  }
  return hipGetLastError();
}

}  // namespace pa

// rope_kv_append: rotary position encoding of the new tokens' Q and K, fused with the
// append of K and V into their pages.
//
// The attention sub-layer turns Q and K by the token's position before attention
// ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §Llama 3.2 1B架构拆解), and a token's
// K/V joins the page cache before the token attends (same page, §推理流程：从Prefill到Decode).
// Doing both in one pass reads each new row once and writes it once.
//
// Pair i of a head vector is (x[i], x[i + 32]) and turns by the angle pos * f_i, with
// f_i = theta^(-2i/64) or a caller-given table.  Angles are formed and reduced modulo
// 2 pi in fp64 (positions reach tens of thousands of radians), their cosine and sine
// taken in fp64 and rounded to fp32; the rotation itself runs in fp32 and is rounded
// once to bf16.
//
// One workgroup of 256 threads per token.  A head's 64 dims are eight threads' work:
// thread t of a head takes dims 4t .. 4t+3 and 32+4t .. 35+4t (two 8-byte pieces), so
// one load instruction covers eight heads' rows contiguously.  V is copied unchanged.
// Page layouts as for the plain append: K [Hkv][8][bs][8], V [Hkv][64][bs].
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

// sequence s with cu[s] <= t < cu[s+1] (cu ascending, cu[0] = 0)
__device__ __forceinline__ int rope_find_seq(const int32_t* __restrict__ cu, int n_seqs, int t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Rotate four pairs: lo holds dims i..i+3, hi dims i+32..i+35 (bf16 bit pairs).
__device__ __forceinline__ void rotate4(u32x2_t& lo, u32x2_t& hi, const float* c, const float* s) {
  float a[4] = {bf_lo(lo[0]), bf_hi(lo[0]), bf_lo(lo[1]), bf_hi(lo[1])};
  float b[4] = {bf_lo(hi[0]), bf_hi(hi[0]), bf_lo(hi[1]), bf_hi(hi[1])};
  float ra[4], rb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ra[e] = __builtin_fmaf(a[e], c[e], -b[e] * s[e]);
    rb[e] = __builtin_fmaf(b[e], c[e], a[e] * s[e]);
  }
  lo = u32x2_t{pack_bf16x2(ra[0], ra[1]), pack_bf16x2(ra[2], ra[3])};
  hi = u32x2_t{pack_bf16x2(rb[0], rb[1]), pack_bf16x2(rb[2], rb[3])};
}

template <int BS>
__global__ __launch_bounds__(256) void rope_kv_append_kernel(
    const uint16_t* q_in, uint16_t* q_out,  // q_out may be q_in (in place)
    const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, uint16_t* __restrict__ k_pool,
    uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ cu_new_lens, const int32_t* __restrict__ ctx_lens, int n_seqs,
    int num_q_heads, int num_kv_heads, int num_pages, double log2_theta,
    const float* __restrict__ inv_freq) {
  __shared__ float cos_sh[kHeadDim / 2], sin_sh[kHeadDim / 2];
  const int tok = blockIdx.x;
  const int tid = threadIdx.x;
  const int s = rope_find_seq(cu_new_lens, n_seqs, tok);
  const int first = cu_new_lens[s];
  const int n_s = cu_new_lens[s + 1] - first;
  const int pos = ctx_lens[s] - n_s + (tok - first);

  if (tid < kHeadDim / 2) {
    const double f = inv_freq ? (double)inv_freq[tid]
                              : exp2(-(double)(2 * tid) / kHeadDim * log2_theta);
    const double th = (double)pos * f;
    const double r = __builtin_fma(-rint(th / kTwoPi), kTwoPi, th);  // |r| <= pi
    double sn, cn;
    sincos(r, &sn, &cn);
    cos_sh[tid] = (float)cn;
    sin_sh[tid] = (float)sn;
  }
  __syncthreads();
  const int part = tid & 7;  // dims 4 part .. +3 and 32 + 4 part .. +3 of a head
  float c[4], sn[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[e] = cos_sh[4 * part + e];
    sn[e] = sin_sh[4 * part + e];
  }

  // ---- Q: rotated in place or into q_out ---------------------------------------------
  if (q_in) {
    for (int h = tid >> 3; h < num_q_heads; h += 32) {
      const size_t row = ((size_t)tok * num_q_heads + h) * kHeadDim;
      u32x2_t lo = *reinterpret_cast<const u32x2_t*>(q_in + row + 4 * part);
      u32x2_t hi = *reinterpret_cast<const u32x2_t*>(q_in + row + 32 + 4 * part);
      rotate4(lo, hi, c, sn);
      *reinterpret_cast<u32x2_t*>(q_out + row + 4 * part) = lo;
      *reinterpret_cast<u32x2_t*>(q_out + row + 32 + 4 * part) = hi;
    }
  }

  // ---- K rotated and V copied into the token's page slot -------------------------------
  if (pos < 0 || pos >= max_blocks * BS) return;  // inconsistent lengths: drop
  const int page = block_tables[(size_t)s * max_blocks + pos / BS];
  if ((unsigned)page >= (unsigned)num_pages) return;  // bad page id: drop
  const int slot = pos % BS;
  const size_t page_base = (size_t)page * num_kv_heads * (kHeadDim * BS);
  for (int g = tid >> 3; g < num_kv_heads; g += 32) {
    const size_t row = ((size_t)tok * num_kv_heads + g) * kHeadDim;
    u32x2_t lo = *reinterpret_cast<const u32x2_t*>(k_new + row + 4 * part);
    u32x2_t hi = *reinterpret_cast<const u32x2_t*>(k_new + row + 32 + 4 * part);
    rotate4(lo, hi, c, sn);
    // dims 4 part .. +3 sit in 16-byte piece (4 part) / 8 at offset (4 part) % 8
    uint16_t* kh = k_pool + page_base + (size_t)g * (kHeadDim * BS);
    const int d0 = 4 * part, d1 = 32 + 4 * part;
    *reinterpret_cast<u32x2_t*>(kh + ((d0 >> 3) * BS + slot) * 8 + (d0 & 7)) = lo;
    *reinterpret_cast<u32x2_t*>(kh + ((d1 >> 3) * BS + slot) * 8 + (d1 & 7)) = hi;
  }
  for (int e = tid; e < num_kv_heads * kHeadDim; e += 256) {
    const int g = e / kHeadDim, i = e - g * kHeadDim;
    v_pool[page_base + ((size_t)g * kHeadDim + i) * BS + slot] =
        v_new[(size_t)tok * num_kv_heads * kHeadDim + e];
  }
}

}  // namespace

hipError_t launch_rope_kv_append(const LaunchGeom& geo, const void* q_in, void* q_out,
                                 const void* k_new, const void* v_new, void* k_pool,
                                 void* v_pool, const int32_t* block_tables, int max_blocks,
                                 const int32_t* cu_new_lens, const int32_t* ctx_lens,
                                 int n_seqs, int n_new_tokens, double rope_theta,
                                 const float* inv_freq, hipStream_t stream) {
  const dim3 grid(n_new_tokens);
  const dim3 block(256);
  auto* qi = static_cast<const uint16_t*>(q_in);
  auto* qo = static_cast<uint16_t*>(q_out);
  auto* kn = static_cast<const uint16_t*>(k_new);
  auto* vn = static_cast<const uint16_t*>(v_new);
  auto* kp = static_cast<uint16_t*>(k_pool);
  auto* vp = static_cast<uint16_t*>(v_pool);
  const double l2t = inv_freq ? 0.0 : log2(rope_theta);
  if (geo.block_size == 16) {
    hipLaunchKernelGGL(rope_kv_append_kernel<16>, grid, block, 0, stream, qi, qo, kn, vn, kp, vp,
                       block_tables, max_blocks, cu_new_lens, ctx_lens, n_seqs, geo.num_q_heads,
                       geo.num_kv_heads, geo.num_pages, l2t, inv_freq);
  } else {
    hipLaunchKernelGGL(rope_kv_append_kernel<32>, grid, block, 0, stream, qi, qo, kn, vn, kp, vp,
                       block_tables, max_blocks, cu_new_lens, ctx_lens, n_seqs, geo.num_q_heads,
                       geo.num_kv_heads, geo.num_pages, l2t, inv_freq);
  }
  return hipGetLastError();
}

}  // namespace pa

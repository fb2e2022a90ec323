// Bandwidth-bound element-wise steps of a decoder layer: residual add fused with RMS
// normalisation, and the SiLU-gated product of the MLP.
//
// Every sub-layer is wrapped in RMS normalisation and a residual connection, and the MLP
// multiplies SiLU of the gate projection with the up projection
// ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §Llama 3.2 1B架构拆解); fusing the residual add
// into the normalisation and the activation into the product keeps each activation row
// to one pass through memory ("Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎", §算子融合).
//
// residual_rmsnorm: one wave per row, four rows per 256-thread workgroup.  A lane holds up
// to NC 16-byte chunks of its row in registers (chunk lane + 64 i), so the row is read once
// and all of its loads are in flight together: h = x + r (fp32, rounded to bf16 and stored
// as the next residual), the sum of h^2 over the row (a DPP reduction inside the wave, no
// barrier), out = h * 1/sqrt(mean + eps) * gamma rounded once to bf16.
// silu_mul: a workgroup per (row, group of 256 U chunks); all 2U loads of a thread are
// issued before the first product: out = g / (1 + e^-g) * u in fp32.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kMaxNormChunks = 16;  // 16-byte chunks per lane: rows up to 64 * 16 * 8 = 8192

template <bool RES, int NC>
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* r_in, uint16_t* r_out,  // r may be in place
    const uint16_t* __restrict__ gamma, uint16_t* __restrict__ out, int n_rows, int hidden,
    float eps) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // wave-uniform, and the kernel has no workgroup barrier
  const int lane = threadIdx.x & 63;
  const int chunks = hidden >> 3;
  const size_t base = (size_t)row * hidden;
  // gamma joins the first batch of loads for rows of up to 2048; wider rows load it after
  // the reduction, to keep the register count (and the occupancy) in bounds
  constexpr bool kEarlyGamma = NC <= 4;
  u32x4_t h[NC], b[NC], gm[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    h[i] = b[i] = gm[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (c < chunks) {
      h[i] = *reinterpret_cast<const u32x4_t*>(x + base + 8 * c);
      if constexpr (RES) b[i] = *reinterpret_cast<const u32x4_t*>(r_in + base + 8 * c);
      if constexpr (kEarlyGamma) gm[i] = *reinterpret_cast<const u32x4_t*>(gamma + 8 * c);
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c >= chunks) continue;
    if constexpr (RES) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        h[i][w] = pack_bf16x2(bf_lo(h[i][w]) + bf_lo(b[i][w]), bf_hi(h[i][w]) + bf_hi(b[i][w]));
      *reinterpret_cast<u32x4_t*>(r_out + base + 8 * c) = h[i];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = bf_lo(h[i][w]), hi = bf_hi(h[i][w]);
      ss = __builtin_fmaf(lo, lo, ss);
      ss = __builtin_fmaf(hi, hi, ss);
    }
  }
  const float inv = 1.f / sqrtf(wave_sum(ss) / (float)hidden + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + 64 * i;
    if (c >= chunks) continue;
    if constexpr (!kEarlyGamma) gm[i] = *reinterpret_cast<const u32x4_t*>(gamma + 8 * c);
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o[w] = pack_bf16x2(bf_lo(h[i][w]) * inv * bf_lo(gm[i][w]),
                         bf_hi(h[i][w]) * inv * bf_hi(gm[i][w]));
    *reinterpret_cast<u32x4_t*>(out + base + 8 * c) = o;
  }
}

__device__ __forceinline__ float silu_times(float g, float u) {
  return g / (1.f + __expf(-g)) * u;
}

template <int U>
__global__ __launch_bounds__(256) void silu_mul_kernel(
    const uint16_t* __restrict__ gate, const uint16_t* __restrict__ up, int64_t ld_in,
    uint16_t* __restrict__ out, int64_t ld_out, int width) {
  const int64_t row = blockIdx.x;
  const int cpr = width >> 3;  // 16-byte chunks per row
  const int c0 = blockIdx.y * (256 * U) + threadIdx.x;
  const uint16_t* g = gate + row * ld_in;
  const uint16_t* u = up + row * ld_in;
  uint16_t* o = out + row * ld_out;
  u32x4_t gv[U], uv[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int c = c0 + 256 * j;
    gv[j] = uv[j] = u32x4_t{0u, 0u, 0u, 0u};
    if (c < cpr) {
      gv[j] = *reinterpret_cast<const u32x4_t*>(g + 8 * c);
      uv[j] = *reinterpret_cast<const u32x4_t*>(u + 8 * c);
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int c = c0 + 256 * j;
    if (c >= cpr) continue;
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      r[w] = pack_bf16x2(silu_times(bf_lo(gv[j][w]), bf_lo(uv[j][w])),
                         silu_times(bf_hi(gv[j][w]), bf_hi(uv[j][w])));
    *reinterpret_cast<u32x4_t*>(o + 8 * c) = r;
  }
}

template <bool RES>
void launch_norm_rows(const uint16_t* x, const uint16_t* ri, uint16_t* ro, const uint16_t* gm,
                      uint16_t* o, int n_rows, int hidden, float eps, hipStream_t stream) {
  const dim3 grid((n_rows + 3) / 4), block(256);
  const int per_lane = (hidden / 8 + 63) / 64;
  if (per_lane <= 4)
    hipLaunchKernelGGL((residual_rmsnorm_kernel<RES, 4>), grid, block, 0, stream, x, ri, ro, gm, o,
                       n_rows, hidden, eps);
  else if (per_lane <= 8)
    hipLaunchKernelGGL((residual_rmsnorm_kernel<RES, 8>), grid, block, 0, stream, x, ri, ro, gm, o,
                       n_rows, hidden, eps);
  else
    hipLaunchKernelGGL((residual_rmsnorm_kernel<RES, kMaxNormChunks>), grid, block, 0, stream, x,
                       ri, ro, gm, o, n_rows, hidden, eps);
}

}  // namespace

int rmsnorm_max_hidden() { return 64 * kMaxNormChunks * 8; }

int silu_max_width() { return 1 << 24; }  // 8192 groups of 256 chunks on grid axis y

hipError_t launch_residual_rmsnorm(const void* x, const void* residual_in, void* residual_out,
                                   const void* gamma, void* out, int n_rows, int hidden,
                                   float eps, hipStream_t stream) {
  auto* xi = static_cast<const uint16_t*>(x);
  auto* ri = static_cast<const uint16_t*>(residual_in);
  auto* ro = static_cast<uint16_t*>(residual_out);
  auto* gm = static_cast<const uint16_t*>(gamma);
  auto* o = static_cast<uint16_t*>(out);
  if (residual_in)
    launch_norm_rows<true>(xi, ri, ro, gm, o, n_rows, hidden, eps, stream);
  else
    launch_norm_rows<false>(xi, ri, ro, gm, o, n_rows, hidden, eps, stream);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void* gate, const void* up, int64_t ld_in, void* out,
                           int64_t ld_out, int n_rows, int width, int compute_units,
                           hipStream_t stream) {
  // Four chunks per thread keep eight 16-byte loads in flight; with too few rows to fill
  // the chip that way, one chunk per thread spreads a row over four times the workgroups.
  const int cpr = width / 8;
  auto* g = static_cast<const uint16_t*>(gate);
  auto* u = static_cast<const uint16_t*>(up);
  auto* o = static_cast<uint16_t*>(out);
  const int64_t wide_wgs = (int64_t)n_rows * ((cpr + 1023) / 1024);
  if (wide_wgs >= 4 * (int64_t)std::max(compute_units, 1)) {
    hipLaunchKernelGGL(silu_mul_kernel<4>, dim3(n_rows, (cpr + 1023) / 1024), dim3(256), 0, stream,
                       g, u, ld_in, o, ld_out, width);
  } else {
    hipLaunchKernelGGL(silu_mul_kernel<1>, dim3(n_rows, (cpr + 255) / 256), dim3(256), 0, stream,
                       g, u, ld_in, o, ld_out, width);
  }
  return hipGetLastError();
}

}  // namespace pa

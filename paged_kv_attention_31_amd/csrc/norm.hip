// Bandwidth-bound element-wise steps of a decoder layer: residual add fused with RMS
// normalisation, and the SiLU-gated product of the MLP.
//
// Every sub-layer is wrapped in RMS normalisation and a residual connection, and the MLP
// multiplies SiLU of the gate projection with the up projection
// ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §Llama 3.2 1B架构拆解); fusing the residual add
// into the normalisation and the activation into the product keeps each activation row
// to one pass through memory ("Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎", §算子融合).
//
// residual_rmsnorm: a wave normalises whole rows, four waves per 256-thread workgroup.  A
// lane holds up to NC 16-byte chunks of a row in registers (chunk lane + 64 i), so a row is
// read once and all of its loads are in flight together: h = x + r (fp32, rounded to bf16
// and stored as the next residual), the sum of h^2 over the row (a DPP reduction inside
// the wave, no barrier), out = h * 1/sqrt(mean + eps) * gamma rounded once to bf16.  Rows
// of up to 4096 go grid-stride over one workgroup per compute unit, the next row's loads
// issued before the current row's arithmetic and stores, so reads and writes overlap in
// every wave; wider rows fill the registers with one row, and a wave takes a single row.
// Rows are reached through buffer descriptors sized to the row (empty past the last row):
// every load and store is issued unconditionally, which keeps the compiler's memory wait
// counts exact across the loop.
// silu_mul: a workgroup per (row, group of 256 U chunks); all 2U loads of a thread are
// issued before the first product: out = g / (1 + e^-g) * u in fp32.
// Both kernels read their activations once, with nontemporal loads; their outputs are
// stored as usual, for the kernel that reads them next.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kMaxNormChunks = 16;  // 16-byte chunks per lane: rows up to 64 * 16 * 8 = 8192

constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3: raw (untyped) access
constexpr int kNontemporal = 2;         // cache policy of a buffer access: nt (read once)

// A descriptor over one row of n_bytes (0 past the last row): loads outside it return zeros
// and stores outside it are dropped, so every lane issues every load and store.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint16_t* p, int n_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, n_bytes, kRsrcWord3);
}

// Rows of up to 4096 (8 chunks per lane) keep two rows in registers and prefetch.
template <int NC>
constexpr bool kNormPrefetch = NC <= 8;

template <bool RES, int NC>
struct NormRow {
  u32x4_t h[NC], b[NC];
};

// Issues the loads of x and r of one row (chunk lane + 64 i of the row in h[i], b[i]).
template <bool RES, int NC>
__device__ __forceinline__ void norm_load(NormRow<RES, NC>& v, __amdgpu_buffer_rsrc_t rx,
                                          __amdgpu_buffer_rsrc_t rr, int lane) {
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    v.h[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (lane + 64 * i) * 16, 0, kNontemporal);
    if constexpr (RES)
      v.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rr, (lane + 64 * i) * 16, 0, kNontemporal);
  }
}

// h = x + r (stored as the next residual), then out = h / sqrt(mean(h^2) + eps) * gamma.
// Chunks past the row end hold zeros and add nothing to the sum of squares.
template <bool RES, int NC, bool kEarlyGamma>
__device__ __forceinline__ void norm_store(NormRow<RES, NC>& v, u32x4_t (&gm)[NC],
                                           __amdgpu_buffer_rsrc_t rg, __amdgpu_buffer_rsrc_t rro,
                                           __amdgpu_buffer_rsrc_t ro, int lane, int hidden,
                                           float eps) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if constexpr (RES) {
#pragma unroll
      for (int w = 0; w < 4; ++w)
        v.h[i][w] = pack_bf16x2(bf_lo(v.h[i][w]) + bf_lo(v.b[i][w]),
                                bf_hi(v.h[i][w]) + bf_hi(v.b[i][w]));
      __builtin_amdgcn_raw_buffer_store_b128(v.h[i], rro, (lane + 64 * i) * 16, 0, 0);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = bf_lo(v.h[i][w]), hi = bf_hi(v.h[i][w]);
      ss = __builtin_fmaf(lo, lo, ss);
      ss = __builtin_fmaf(hi, hi, ss);
    }
  }
  const float inv = 1.f / sqrtf(wave_sum(ss) / (float)hidden + eps);
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    if constexpr (!kEarlyGamma)
      gm[i] = __builtin_amdgcn_raw_buffer_load_b128(rg, (lane + 64 * i) * 16, 0, 0);
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o[w] = pack_bf16x2(bf_lo(v.h[i][w]) * inv * bf_lo(gm[i][w]),
                         bf_hi(v.h[i][w]) * inv * bf_hi(gm[i][w]));
    __builtin_amdgcn_raw_buffer_store_b128(o, ro, (lane + 64 * i) * 16, 0, 0);
  }
}

template <bool RES, int NC>
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(
    const uint16_t* __restrict__ x, const uint16_t* r_in, uint16_t* r_out,  // r may be in place
    const uint16_t* __restrict__ gamma, uint16_t* __restrict__ out, int n_rows, int hidden,
    float eps) {
  const int64_t stride = (int64_t)gridDim.x * 4;  // waves in the grid
  const int row0 = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (row0 >= n_rows) return;  // wave-uniform, and the kernel has no workgroup barrier
  int64_t row = row0;  // 64-bit: the prefetch's rows past the last one never wrap around
  const int lane = threadIdx.x & 63;
  const int row_bytes = hidden * 2;
  // gamma is loaded once per wave for rows of up to 2048; wider rows load it after each
  // reduction, to keep the register count in bounds
  constexpr bool kEarlyGamma = NC <= 4;
  const __amdgpu_buffer_rsrc_t rg = row_rsrc(gamma, row_bytes);
  u32x4_t gm[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i)
    gm[i] = kEarlyGamma ? __builtin_amdgcn_raw_buffer_load_b128(rg, (lane + 64 * i) * 16, 0, 0)
                        : u32x4_t{0u, 0u, 0u, 0u};
  // past the last row the descriptors are empty: loads return zeros, stores are dropped
  auto load = [&](NormRow<RES, NC>& v, int64_t r) {
    const bool live = r < n_rows;
    const size_t off = (size_t)(live ? r : 0) * hidden;
    const int n = live ? row_bytes : 0;
    norm_load<RES, NC>(v, row_rsrc(x + off, n), row_rsrc(RES ? r_in + off : x, n), lane);
  };
  auto store = [&](NormRow<RES, NC>& v, int64_t r) {
    const bool live = r < n_rows;
    const size_t off = (size_t)(live ? r : 0) * hidden;
    const int n = live ? row_bytes : 0;
    norm_store<RES, NC, kEarlyGamma>(v, gm, rg, row_rsrc(RES ? r_out + off : out, n),
                                     row_rsrc(out + off, n), lane, hidden, eps);
  };
  NormRow<RES, NC> va;
  if constexpr (!kNormPrefetch<NC>) {  // a row fills the registers: one at a time
    for (; row < n_rows; row += stride) {
      load(va, row);
      store(va, row);
    }
    return;
  } else {
    // Rows row, row + stride, ...: the loads of the next row go out before the arithmetic
    // and the stores of this one, two register sets in turn.  A pass takes two rows with
    // no branch between them (the second may lie past the end), so every load is used in
    // the code that follows it and none is moved later.
    NormRow<RES, NC> vb;
    load(va, row);
    do {
      load(vb, row + stride);
      __builtin_amdgcn_sched_barrier(0);
      store(va, row);
      load(va, row + 2 * stride);
      __builtin_amdgcn_sched_barrier(0);
      store(vb, row + stride);
      row += 2 * stride;
    } while (row < n_rows);
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
      gv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(g + 8 * c));
      uv[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(u + 8 * c));
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

template <bool RES, int NC>
void launch_norm(const uint16_t* x, const uint16_t* ri, uint16_t* ro, const uint16_t* gm,
                 uint16_t* o, int n_rows, int hidden, float eps, int compute_units,
                 hipStream_t stream) {
  // a wave per row; with prefetch, at most one workgroup (four row streams) per compute unit
  int wgs = n_rows / 4 + (n_rows % 4 != 0);
  if (kNormPrefetch<NC>) wgs = std::min(wgs, std::max(compute_units, 1));
  hipLaunchKernelGGL((residual_rmsnorm_kernel<RES, NC>), dim3(wgs), dim3(256), 0, stream, x, ri,
                     ro, gm, o, n_rows, hidden, eps);
}

template <bool RES>
void launch_norm_rows(const uint16_t* x, const uint16_t* ri, uint16_t* ro, const uint16_t* gm,
                      uint16_t* o, int n_rows, int hidden, float eps, int compute_units,
                      hipStream_t stream) {
  const int per_lane = (hidden / 8 + 63) / 64;
  if (per_lane <= 4)
    launch_norm<RES, 4>(x, ri, ro, gm, o, n_rows, hidden, eps, compute_units, stream);
  else if (per_lane <= 8)
    launch_norm<RES, 8>(x, ri, ro, gm, o, n_rows, hidden, eps, compute_units, stream);
  else
    launch_norm<RES, kMaxNormChunks>(x, ri, ro, gm, o, n_rows, hidden, eps, compute_units,
                                     stream);
}

}  // namespace

int rmsnorm_max_hidden() { return 64 * kMaxNormChunks * 8; }

int silu_max_width() { return 1 << 24; }  // 8192 groups of 256 chunks on grid axis y

hipError_t launch_residual_rmsnorm(const void* x, const void* residual_in, void* residual_out,
                                   const void* gamma, void* out, int n_rows, int hidden,
                                   float eps, int compute_units, hipStream_t stream) {
  auto* xi = static_cast<const uint16_t*>(x);
  auto* ri = static_cast<const uint16_t*>(residual_in);
  auto* ro = static_cast<uint16_t*>(residual_out);
  auto* gm = static_cast<const uint16_t*>(gamma);
  auto* o = static_cast<uint16_t*>(out);
  if (residual_in)
    launch_norm_rows<true>(xi, ri, ro, gm, o, n_rows, hidden, eps, compute_units, stream);
  else
    launch_norm_rows<false>(xi, ri, ro, gm, o, n_rows, hidden, eps, compute_units, stream);
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

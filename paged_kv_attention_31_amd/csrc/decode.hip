// pa_decode: one query token per sequence attends to the sequence's paged K/V.
//
// The method ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §PagedAttention and
// §在线Softmax; "Tiny-vLLM 实战", §算子融合): keys are read page by page through the
// block table, and softmax runs in one pass with a running maximum and a running sum
// that is rescaled whenever the maximum grows.  Decode moves every KV byte once and
// does 4 flop per byte, so the kernel is bound by HBM bandwidth (same guide,
// §推理流程: decode is memory-bound); everything below is arranged around streaming
// the pages with wide coalesced loads.
//
// Work split: one workgroup (4 waves) per (sequence, KV head, KV partition).  The four
// query heads of the KV head share every K/V byte the workgroup reads.  A wave takes
// 64-token tiles of the partition (tiles w, w+4, ...):
//   scores:  lane t owns token t of the tile.  The K page layout [Hkv][8][bs][8] makes
//            "lane t reads piece c of token t" a contiguous run over lanes, so eight
//            16-byte loads per lane bring the lane its token's whole K row.  q (4 heads,
//            bf16) sits in LDS and is read as 16-byte broadcasts; dot products use
//            v_dot2c_f32_bf16 (two bf16 products per instruction, fp32 accumulate).
//   softmax: per head a wave max (DPP inside 16-lane rows, readlane across rows), scores
//            pre-scaled by scale*log2(e) so exponentials are exp2; the probabilities are
//            rounded to bf16 and go to LDS.
//   P.V:     the V page layout [Hkv][64][bs] gives each lane 8 consecutive tokens of one
//            dimension per 16-byte load, i.e. bf16 pairs along the token axis, so P.V is
//            again v_dot2c_f32_bf16 (fp32 accumulate) against the lane's 8 probabilities.  Tokens past the end of the context are excluded
//            by selection, never by multiplying by a zero weight, so stale pool bytes
//            (even NaN) cannot leak.
// At the end the 4 waves merge their (max, sum, output) through LDS.  With one
// partition the workgroup writes the normalised bf16 row; otherwise it writes fp32
// partials and decode_merge_kernel combines partitions in ascending order (fixed order:
// results do not depend on scheduling).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

template <int BS>
__global__ __launch_bounds__(256) void decode_part_kernel(
    uint16_t* __restrict__ out, float* __restrict__ ws_o, float2* __restrict__ ws_ml,
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
    int max_blocks, const int32_t* __restrict__ ctx_lens, int num_pages, int num_kv_heads,
    int n_parts, int part_tokens, float qk_scale) {
  constexpr int LPR = BS / 8;    // lanes sharing one V row (one head dimension)
  constexpr int RPI = 64 / LPR;  // V rows covered by one 16-byte-per-lane load
  constexpr int PPT = 64 / BS;   // pages per 64-token tile
  constexpr int NV = LPR;        // head dimensions each lane accumulates

  const int bid = blockIdx.x;
  const int part = bid % n_parts;
  const int sg = bid / n_parts;
  const int g = sg % num_kv_heads;
  const int s = sg / num_kv_heads;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int hq = num_kv_heads * kGroup;

  int ctx = ctx_lens[s];
  ctx = max(0, min(min(ctx, max_blocks * BS), n_parts * part_tokens));
  const int p0 = part * part_tokens;
  const int p1 = min(ctx, p0 + part_tokens);
  if (n_parts > 1 && p0 >= ctx) return;  // partition past the end: the merge skips it

  __shared__ uint4 q_sh[kGroup][8];                // [head][piece], bf16 x 8
  __shared__ __attribute__((aligned(16))) uint16_t p_sh[kDecodeWaves][kGroup][64];  // bf16 p
  __shared__ float red_m[kDecodeWaves][kGroup];
  __shared__ float red_l[kDecodeWaves][kGroup];
  __shared__ float red_o[kDecodeWaves][kGroup][64];
  __shared__ int bad_sh;

  if (tid < kGroup * 8) {
    q_sh[tid >> 3][tid & 7] =
        reinterpret_cast<const uint4*>(q + ((size_t)s * hq + g * kGroup) * kHeadDim)[tid];
  }
  if (tid == 0) bad_sh = 0;
  __syncthreads();

  const int32_t* bt = block_tables + (size_t)s * max_blocks;
  const size_t head_stride = (size_t)kHeadDim * BS;  // elements of one (page, head)
  const size_t page_stride = head_stride * num_kv_heads;
  const uint16_t* k_head = k_pool + g * head_stride;
  const uint16_t* v_head = v_pool + g * head_stride + (lane / LPR) * BS + (lane % LPR) * 8;

  float m[kGroup], l[kGroup], acc[NV][kGroup];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i][h] = 0.f;
  }
  int bad = 0;

  const int n_tiles = p1 > p0 ? (p1 - p0 + 63) / 64 : 0;
  for (int ti = w; ti < n_tiles; ti += kDecodeWaves) {
    const int t0 = p0 + ti * 64;
    const int nvalid = min(64, p1 - t0);
    const int last_blk = (p1 - 1) / BS;

    // ---- K: lane owns one token --------------------------------------------------------
    const int pos = t0 + min(lane, nvalid - 1);
    int kpage = bt[pos / BS];
    if ((unsigned)kpage >= (unsigned)num_pages) { bad = 1; kpage = 0; }
    const uint16_t* kb = k_head + (size_t)kpage * page_stride + (pos % BS) * 8;
    uint4 kc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) kc[c] = *reinterpret_cast<const uint4*>(kb + c * BS * 8);

    // ---- V: lane owns 8 consecutive tokens of NV dimensions, per page ----------------
    uint4 vc[PPT][NV];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      int vpage = bt[min(t0 / BS + j, last_blk)];
      if ((unsigned)vpage >= (unsigned)num_pages) { bad = 1; vpage = 0; }
      const uint16_t* vb = v_head + (size_t)vpage * page_stride;
#pragma unroll
      for (int i = 0; i < NV; ++i) vc[j][i] = *reinterpret_cast<const uint4*>(vb + i * RPI * BS);
    }

    // ---- scores ------------------------------------------------------------------------
    // q is re-read from LDS every tile as 16-byte broadcasts, one piece ahead of its use;
    // the opaque zero offset and the scheduling fences keep the compiler from hoisting
    // all 32 reads (128 registers) out of the loop.
    int qofs = 0;
    asm volatile("" : "+s"(qofs));
    const uint4* qrow = &q_sh[0][0] + qofs;
    float x[kGroup] = {0.f, 0.f, 0.f, 0.f};
    uint4 qn[kGroup];
#pragma unroll
    for (int h = 0; h < kGroup; ++h) qn[h] = qrow[h * 8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 qc[kGroup];
#pragma unroll
      for (int h = 0; h < kGroup; ++h) qc[h] = qn[h];
      if (c + 1 < 8) {
#pragma unroll
        for (int h = 0; h < kGroup; ++h) qn[h] = qrow[h * 8 + c + 1];
      }
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        float a = x[h];
        a = dot2(kc[c].x, qc[h].x, a);
        a = dot2(kc[c].y, qc[h].y, a);
        a = dot2(kc[c].z, qc[h].z, a);
        a = dot2(kc[c].w, qc[h].w, a);
        x[h] = a;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int h = 0; h < kGroup; ++h) x[h] = lane < nvalid ? x[h] * qk_scale : kNegInf;

    // ---- online softmax update ---------------------------------------------------------
    // p is rounded to bf16 once; the same rounded value feeds both the running sum and
    // the P.V product, so the output is an exact convex combination of the V rows.
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const float mt = wave_max(x[h]);
      const float mn = fmaxf(m[h], mt);
      const float alpha = fast_exp2(m[h] - mn);  // 0 on the first tile (m = -inf)
      const uint16_t pb = to_bf16(fast_exp2(x[h] - mn));  // 0 for tokens past the end
      l[h] = l[h] * alpha + __uint_as_float((uint32_t)pb << 16);
      m[h] = mn;
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i][h] *= alpha;
      p_sh[w][h][lane] = pb;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- P.V: two tokens per v_dot2c_f32_bf16 -------------------------------------------
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int tb = j * BS + (lane % LPR) * 8;  // tile index of this lane's first token
      uint4 pp[kGroup];
#pragma unroll
      for (int h = 0; h < kGroup; ++h) pp[h] = *reinterpret_cast<const uint4*>(&p_sh[w][h][tb]);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        uint4 vv = vc[j][i];
        if (nvalid < 64) {
          // tokens past the end may hold stale bytes (even NaN): clear them
          uint32_t wv[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (tb + k >= nvalid) wv[k >> 1] &= (k & 1) ? 0x0000ffffu : 0xffff0000u;
          }
          vv = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
#pragma unroll
        for (int h = 0; h < kGroup; ++h) {
          float a = acc[i][h];
          a = dot2(vv.x, pp[h].x, a);
          a = dot2(vv.y, pp[h].y, a);
          a = dot2(vv.z, pp[h].z, a);
          a = dot2(vv.w, pp[h].w, a);
          acc[i][h] = a;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge lanes, then waves -------------------------------------------------------------
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    l[h] = wave_sum(l[h]);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float a = acc[i][h];
      a += shfl_xor_f(a, 1);
      if (LPR == 4) a += shfl_xor_f(a, 2);
      acc[i][h] = a;
    }
  }
  if (lane % LPR == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
#pragma unroll
      for (int i = 0; i < NV; ++i) red_o[w][h][i * RPI + lane / LPR] = acc[i][h];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      red_m[w][h] = m[h];
      red_l[w][h] = l[h];
    }
  }
  if (bad) bad_sh = 1;
  __syncthreads();

  const int h = tid >> 6;
  const int d = tid & 63;
  float M = kNegInf;
#pragma unroll
  for (int v = 0; v < kDecodeWaves; ++v) M = fmaxf(M, red_m[v][h]);
  float L = 0.f, O = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int v = 0; v < kDecodeWaves; ++v) {
      const float mv = red_m[v][h];
      if (mv != kNegInf) {
        const float f = fast_exp2(mv - M);
        L += red_l[v][h] * f;
        O += red_o[v][h][d] * f;
      }
    }
  }
  if (bad_sh) O = __builtin_nanf("");
  const int head = g * kGroup + h;
  if (n_parts == 1) {
    out[((size_t)s * hq + head) * kHeadDim + d] = to_bf16(L > 0.f ? O / L : O * 0.f);
  } else {
    const size_t slot = ((size_t)s * n_parts + part) * hq + head;
    ws_o[slot * kHeadDim + d] = O;
    if (d == 0) ws_ml[slot] = make_float2(M, L);
  }
}

// Combine partition partials of one (sequence, KV head): M = max_j m_j,
// L = sum_j l_j 2^(m_j - M), out = sum_j o_j 2^(m_j - M) / L, j ascending.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_o, const float2* __restrict__ ws_ml,
    const int32_t* __restrict__ ctx_lens, int max_tokens, int num_kv_heads, int n_parts,
    int part_tokens) {
  const int g = blockIdx.x % num_kv_heads;
  const int s = blockIdx.x / num_kv_heads;
  const int hq = num_kv_heads * kGroup;
  const int head = g * kGroup + (threadIdx.x >> 6);
  const int d = threadIdx.x & 63;
  int ctx = ctx_lens[s];
  ctx = max(0, min(ctx, max_tokens));
  const int np = (ctx + part_tokens - 1) / part_tokens;
  float M = kNegInf;
  for (int j = 0; j < np; ++j) M = fmaxf(M, ws_ml[((size_t)s * n_parts + j) * hq + head].x);
  float L = 0.f, O = 0.f;
  for (int j = 0; j < np; ++j) {
    const size_t slot = ((size_t)s * n_parts + j) * hq + head;
    const float2 ml = ws_ml[slot];
    if (ml.x != kNegInf) {
      const float f = fast_exp2(ml.x - M);
      L += ml.y * f;
      O += ws_o[slot * kHeadDim + d] * f;
    }
  }
  out[((size_t)s * hq + head) * kHeadDim + d] = to_bf16(L > 0.f ? O / L : O * 0.f);
}

}  // namespace

size_t decode_workspace_bytes(int n_seqs, int n_parts, int num_q_heads) {
  if (n_parts <= 1) return 0;
  const size_t slots = (size_t)n_seqs * n_parts * num_q_heads;
  return slots * kHeadDim * sizeof(float) + slots * sizeof(float2);
}

hipError_t launch_decode(const LaunchGeom& geo, void* out, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables, int max_blocks,
                         const int32_t* ctx_lens, int n_seqs, int n_parts, int part_tokens,
                         float scale, void* workspace, hipStream_t stream) {
  const float qk_scale = scale * kLog2e;
  float* ws_o = nullptr;
  float2* ws_ml = nullptr;
  if (n_parts > 1) {
    const size_t slots = (size_t)n_seqs * n_parts * geo.num_q_heads;
    ws_o = static_cast<float*>(workspace);
    ws_ml = reinterpret_cast<float2*>(ws_o + slots * kHeadDim);
  }
  const dim3 grid((unsigned)((size_t)n_seqs * geo.num_kv_heads * n_parts));
  const dim3 block(256);
  auto* o = static_cast<uint16_t*>(out);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kp = static_cast<const uint16_t*>(k_pool);
  auto* vp = static_cast<const uint16_t*>(v_pool);
  if (geo.block_size == 16) {
    hipLaunchKernelGGL(decode_part_kernel<16>, grid, block, 0, stream, o, ws_o, ws_ml, qq, kp, vp,
                       block_tables, max_blocks, ctx_lens, geo.num_pages, geo.num_kv_heads,
                       n_parts, part_tokens, qk_scale);
  } else {
    hipLaunchKernelGGL(decode_part_kernel<32>, grid, block, 0, stream, o, ws_o, ws_ml, qq, kp, vp,
                       block_tables, max_blocks, ctx_lens, geo.num_pages, geo.num_kv_heads,
                       n_parts, part_tokens, qk_scale);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_parts == 1) return e;
  const dim3 mgrid((unsigned)((size_t)n_seqs * geo.num_kv_heads));
  const int max_tokens = (int)std::min<int64_t>((int64_t)max_blocks * geo.block_size,
                                                  (int64_t)n_parts * part_tokens);
  hipLaunchKernelGGL(decode_merge_kernel, mgrid, block, 0, stream, o, ws_o, ws_ml, ctx_lens,
                     max_tokens, geo.num_kv_heads, n_parts, part_tokens);
  return hipGetLastError();
}

}  // namespace pa

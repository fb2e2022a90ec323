// pa_prefill: causal (or full) attention of a prompt, or of a prompt chunk, over paged K/V.
//
// The method: prefill handles all prompt tokens in parallel and is compute-bound
// ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §推理流程：从Prefill到Decode); the
// attention is tiled with online softmax so the seq x seq score matrix never exists
// ("Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎", §算子融合), with a causal mask
// and grouped-query heads (guide, §Llama 3.2 1B架构拆解).  Here Q.K^T and P.V are real
// dense products, so both run on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation (Tiny-vLLM 实战, §CUDA Kernel 优化: bf16 storage, fp32 accumulation).
//
// Work split: one workgroup per (query tile of 32 positions, sequence, KV head); its four
// waves are the four query heads of that KV head and walk the same K/V pages.  Tiles are
// issued longest first (highest query positions see the most keys under the causal mask).
//
// Per wave and per 32-key tile the products are computed transposed:
//   S^T[key][query]  = K . Q^T    A = K rows straight from the K page (the [8][bs][8]
//                                 piece layout gives each lane 16 contiguous bytes),
//                                 B = Q^T, loaded once per workgroup;
//   O^T[dim][query] += V^T . P^T  A = V^T rows from the V page ([64][bs] layout: 2 x 8
//                                 contiguous bytes per lane), B = P^T.
// With the transposed score tile each lane holds whole key columns of one query, so the
// row max and row sum are in-lane reductions plus one exchange between the two
// half-waves, and the MFMA accumulator layout of S^T is already the B-operand layout
// P^T needs (the k index of the PV product runs over the keys in the order the
// accumulator holds them, and the V^T operand is loaded in that same key order).
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kQTile = 32;  // query positions per workgroup
constexpr int kKTile = 32;  // keys per step

// key (tile-relative, 0..15) held by element e (0..7) of the B/A operand for lane half h
__device__ __forceinline__ int pv_key(int h, int e) { return (e < 4 ? 0 : 8) + 4 * h + (e & 3); }

template <int BS>
__global__ __launch_bounds__(256) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ ctx_lens, int n_seqs,
    int n_qtiles, int num_pages, int num_kv_heads, float qk_scale, int causal) {
  const int bid = blockIdx.x;
  const int g = bid % num_kv_heads;
  const int s = (bid / num_kv_heads) % n_seqs;
  const int tile = n_qtiles - 1 - bid / (num_kv_heads * n_seqs);
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int j = lane & 31;    // query column of this lane
  const int half = lane >> 5;
  const int hq = num_kv_heads * kGroup;
  const int head = g * kGroup + w;

  const int qa = cu_q_lens[s];
  const int qlen = cu_q_lens[s + 1] - qa;
  if (tile * kQTile >= qlen) return;
  int ctx = ctx_lens[s];
  ctx = max(0, min(ctx, max_blocks * BS));

  const int qi = tile * kQTile + j;
  const bool qvalid = qi < qlen;
  const int qrow = qa + min(qi, qlen - 1);
  const int qpos = ctx - qlen + min(qi, qlen - 1);          // this lane's query position
  const int pos_first = ctx - qlen + tile * kQTile;          // smallest in the tile
  const int pos_last = ctx - qlen + min(tile * kQTile + kQTile - 1, qlen - 1);
  const int kend = causal ? min(ctx, pos_last + 1) : ctx;    // keys [0, kend)

  // B operand of S^T = K.Q^T: lane (j, half) holds q[j][16*step + 8*half .. +8]
  const uint16_t* qp = q + ((size_t)qrow * hq + head) * kHeadDim + 8 * half;
  bf16x8_t qb[4];
#pragma unroll
  for (int st = 0; st < 4; ++st)
    qb[st] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + 16 * st));

  const int32_t* bt = block_tables + (size_t)s * max_blocks;
  const size_t head_stride = (size_t)kHeadDim * BS;
  const size_t page_stride = head_stride * num_kv_heads;
  const uint16_t* k_head = k_pool + g * head_stride;
  const uint16_t* v_head = v_pool + g * head_stride;
  const int last_blk = kend > 0 ? (kend - 1) / BS : 0;

  float m = kNegInf, lsum = 0.f;
  f32x16_t o0 = {}, o1 = {};
  bool bad = false;

  for (int k0 = 0; k0 < kend; k0 += kKTile) {
    // ---- S^T = K . Q^T --------------------------------------------------------------
    const int key = min(k0 + j, kend - 1);
    int kpage = bt[key / BS];
    if ((unsigned)kpage >= (unsigned)num_pages) { bad = true; kpage = 0; }
    const uint16_t* kb = k_head + (size_t)kpage * page_stride + (key % BS) * 8;
    f32x16_t sacc = {};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint4 a = *reinterpret_cast<const uint4*>(kb + (2 * st + half) * BS * 8);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qb[st],
                                                     sacc, 0, 0, 0);
    }

    // ---- mask, online softmax -----------------------------------------------------------
    float sv[16];
    const bool need_mask = (k0 + kKTile > ctx) || (causal && k0 + kKTile - 1 > pos_first);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = sacc[r] * qk_scale;
      if (need_mask) {
        const int kr = k0 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (kr >= ctx || (causal && kr > qpos)) x = kNegInf;
      }
      sv[r] = x;
    }
    float mt = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sv[r]);
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    const float mn = fmaxf(m, mt);
    const float mref = (mn == kNegInf) ? 0.f : mn;
    const float alpha = fast_exp2(m - mref);
    // p is rounded to bf16 once (the P.V operand); the running sum adds those same
    // rounded values (a dot with (1, 1)), so the normaliser matches the weights used.
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pk[i] = pack_bf16x2(fast_exp2(sv[2 * i] - mref), fast_exp2(sv[2 * i + 1] - mref));
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ps = dot2(pk[i], 0x3F803F80u, ps);
    lsum = lsum * alpha + ps;
    m = mn;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= alpha;
      o1[r] *= alpha;
    }

    // ---- O^T += V^T . P^T ---------------------------------------------------------------
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pb = make_uint4(pk[4 * ks + 0], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]);
      const int kbase = k0 + 16 * ks;  // first key of this k-step (16 keys, one page run)
      int vpage = bt[min(kbase / BS, last_blk)];
      if ((unsigned)vpage >= (unsigned)num_pages) { bad = true; vpage = 0; }
      const uint16_t* vb = v_head + (size_t)vpage * page_stride + (kbase % BS) + 4 * half;
      const bool vtail = kbase + 16 > ctx;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint16_t* row = vb + (size_t)(32 * mb + j) * BS;
        const uint2 lo = *reinterpret_cast<const uint2*>(row);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 8);
        uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
        if (vtail) {
          // keys at or past the end hold stale bytes: zero them (never weight them by 0)
          uint32_t wv[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            if (kbase + pv_key(half, e) >= ctx)
              wv[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          }
          a = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
        if (mb == 0)
          o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, pb), o0, 0,
                                                       0, 0);
        else
          o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, pb), o1, 0,
                                                       0, 0);
      }
    }
  }

  // ---- normalise and store: lane holds dims 8*(r/4) + 4*half + (r%4) of query j ----------
  const float ltot = lsum + shfl_xor_f(lsum, 32);
  float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (bad) inv = __builtin_nanf("");
  if (!qvalid) return;
  uint16_t* op = out + ((size_t)(qa + qi) * hq + head) * kHeadDim + 4 * half;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x16_t& o = mb ? o1 : o0;
      uint2 v;
      v.x = pack_bf16x2(o[4 * r4 + 0] * inv, o[4 * r4 + 1] * inv);
      v.y = pack_bf16x2(o[4 * r4 + 2] * inv, o[4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(op + 32 * mb + 8 * r4) = v;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const LaunchGeom& geo, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables, int max_blocks,
                          const int32_t* cu_q_lens, const int32_t* ctx_lens, int n_seqs,
                          int max_q_len, float scale, int causal, hipStream_t stream) {
  const int n_qtiles = (max_q_len + kQTile - 1) / kQTile;
  const dim3 grid((unsigned)((size_t)n_qtiles * n_seqs * geo.num_kv_heads));
  const dim3 block(256);
  const float qk_scale = scale * kLog2e;
  auto* o = static_cast<uint16_t*>(out);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kp = static_cast<const uint16_t*>(k_pool);
  auto* vp = static_cast<const uint16_t*>(v_pool);
  if (geo.block_size == 16) {
    hipLaunchKernelGGL(prefill_kernel<16>, grid, block, 0, stream, o, qq, kp, vp, block_tables,
                       max_blocks, cu_q_lens, ctx_lens, n_seqs, n_qtiles, geo.num_pages,
                       geo.num_kv_heads, qk_scale, causal);
  } else {
    hipLaunchKernelGGL(prefill_kernel<32>, grid, block, 0, stream, o, qq, kp, vp, block_tables,
                       max_blocks, cu_q_lens, ctx_lens, n_seqs, n_qtiles, geo.num_pages,
                       geo.num_kv_heads, qk_scale, causal);
  }
  return hipGetLastError();
}

}  // namespace pa

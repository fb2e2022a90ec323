// pa_prefill: causal (or full) attention of a prompt, or of a prompt chunk, over paged K/V.
//
// The method: prefill handles all prompt tokens in parallel and is compute-bound
// ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §推理流程：从Prefill到Decode); the
// attention is tiled with online softmax so the seq x seq score matrix never exists
// ("Tiny-vLLM 实战：用 C++/CUDA 手写高性能 LLM 推理引擎", §算子融合), with a causal mask
// and grouped-query heads (guide, §Llama 3.2 1B架构拆解).  Q.K^T and P.V are real dense
// products, so both run on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation
// (Tiny-vLLM 实战, §CUDA Kernel 优化: bf16 storage, fp32 accumulation).
//
// Work split: one workgroup per (query tile of 32 positions, sequence, KV head); its four
// waves are the four query heads of that KV head.  Tiles are issued longest first (the
// highest query positions see the most keys under the causal mask).
//
// K/V stages: the workgroup copies 64 keys of K and V (the pages' own head slices) from
// HBM into LDS once for all four head-waves, double-buffered: the 256 threads load stage
// s+1 into registers while the waves compute stage s from LDS, then store it to the other
// buffer.  K keeps the page's [8 pieces][bs][8] order (a wave's A-operand reads are then
// contiguous 512-byte runs); V rows ([64 dims][bs]) are padded by 8 bytes so the 32 rows
// an MFMA A-operand read touches fall in distinct LDS banks.  V values of keys past the
// context are zeroed while staging, so stale pool bytes (even NaN) never reach P.V.
//
// Per wave and per 32 keys the products are computed transposed:
//   S^T[key][query]  = K . Q^T    A = K rows from LDS, B = Q^T (registers, loaded once);
//   O^T[dim][query] += V^T . P^T  A = V^T rows from LDS,  B = P^T.
// With the transposed score tile each lane holds 16 keys of one query, so the row max
// and row sum are in-lane reductions plus one exchange between the two half-waves
// (v_permlane32_swap), and the MFMA accumulator layout of S^T is already the B-operand
// layout P^T needs (the k index of the PV product runs over the keys in the order the
// accumulator holds them, and the V^T operand is read in that same key order).
// scale * log2(e) is folded into one FMA ahead of exp2; the output is rescaled only when
// some row's running maximum grew.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kQTile = 32;   // query positions per workgroup
constexpr int kStage = 64;   // keys per LDS stage
constexpr int kThreads = 256;

// Own value and the value of lane j ^ 32 (the two half-waves hold the same query's
// keys), in either order, from one v_permlane32_swap (it exchanges the upper half of its
// first operand with the lower half of its second): with both operands equal to x, the
// first is x[j] for j < 32 and x[j - 32] above, the second x[j + 32] below and x[j] above.
// Written as inline asm with both registers in/out: this compiler's builtin for the
// instruction hands back its first result for both.
__device__ __forceinline__ void pair_swap(float x, float& a, float& b) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  unsigned v = u;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(u), "+v"(v));
  a = __builtin_bit_cast(float, u);
  b = __builtin_bit_cast(float, v);
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_swap(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_swap(x, a, b);
  return a + b;  // same two operands in every lane of the pair
}

template <int BS>
struct PrefillLds {
  static constexpr int PPS = kStage / BS;  // pages per stage
  static constexpr int VROW = BS + 4;      // padded V row (elements)
  uint16_t k[2][kStage * kHeadDim];        // [stage][page][8][bs][8]
  uint16_t v[2][PPS][kHeadDim][VROW];      // [stage][page][dim][bs + pad]
};

template <int BS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ ctx_lens, int n_seqs,
    int n_qtiles, int num_pages, int num_kv_heads, float qk_scale, int causal) {
  using Lds = PrefillLds<BS>;
  constexpr int PPS = Lds::PPS;
  constexpr int VROW = Lds::VROW;
  constexpr int KCH = 8 * BS;  // 16-byte chunks of one page's K (or V) head slice
  __shared__ __attribute__((aligned(16))) Lds sh;
  __shared__ int bad_sh;

  const int bid = blockIdx.x;
  const int g = bid % num_kv_heads;
  const int s = (bid / num_kv_heads) % n_seqs;
  const int tile = n_qtiles - 1 - bid / (num_kv_heads * n_seqs);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
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
  const int n_stages = (kend + kStage - 1) / kStage;
  const int last_blk = kend > 0 ? (kend - 1) / BS : 0;

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

  // ---- staging: thread t moves K chunks t, t+256 and V chunks t, t+256 of a stage ------
  // chunk c of a stage: page c / KCH, 16-byte piece c % KCH of that page's head slice.
  bool bad = false;
  uint4 kr0, kr1, vr0, vr1;  // the thread's two K and two V chunks of the next stage
  auto chunk_base = [&](int k0, int c) -> size_t {
    const int pj = c / KCH;
    int pid = bt[min(k0 / BS + pj, last_blk)];
    if ((unsigned)pid >= (unsigned)num_pages) { bad = true; pid = 0; }
    return (size_t)pid * page_stride + (size_t)(c - pj * KCH) * 8;
  };
  auto stage_load = [&](int st) {
    const int k0 = st * kStage;
    const size_t b0 = chunk_base(k0, tid);
    const size_t b1 = chunk_base(k0, tid + kThreads);
    kr0 = *reinterpret_cast<const uint4*>(k_head + b0);
    vr0 = *reinterpret_cast<const uint4*>(v_head + b0);
    kr1 = *reinterpret_cast<const uint4*>(k_head + b1);
    vr1 = *reinterpret_cast<const uint4*>(v_head + b1);
  };
  // V chunk c: dim row within / (BS/8), keys 8 * (within % (BS/8)) .. +8 of page c / KCH;
  // keys at or past the context end are cleared
  auto store_v = [&](int k0, int c, uint4 vv, int buf) {
    const int pj = c / KCH;
    const int within = c - pj * KCH;
    const int row = within / (BS / 8);
    const int c8 = within - row * (BS / 8);
    const int key0 = k0 + pj * BS + c8 * 8;
    if (key0 + 8 > ctx) {
      uint32_t wv[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (key0 + e >= ctx) wv[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      }
      vv = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    uint16_t* dst = &sh.v[buf][pj][row][c8 * 8];
    *reinterpret_cast<uint2*>(dst) = make_uint2(vv.x, vv.y);
    *reinterpret_cast<uint2*>(dst + 4) = make_uint2(vv.z, vv.w);
  };
  auto stage_store = [&](int st, int buf) {
    const int k0 = st * kStage;
    *reinterpret_cast<uint4*>(&sh.k[buf][tid * 8]) = kr0;
    *reinterpret_cast<uint4*>(&sh.k[buf][(tid + kThreads) * 8]) = kr1;
    store_v(k0, tid, vr0, buf);
    store_v(k0, tid + kThreads, vr1, buf);
  };

  float m = kNegInf, lsum = 0.f;  // this lane's query row: running max (scaled) and sum
  f32x16_t o0 = {}, o1 = {};

  // one 32-key half of a stage: keys k0 + 32 * hh .. +32
  auto compute_half = [&](int buf, int k0, int hh) {
    const int kb = k0 + 32 * hh;
    // ---- S^T = K . Q^T ------------------------------------------------------------------
    const int kk = 32 * hh + j;  // key within the stage held as A row by this lane
    const uint16_t* krow =
        &sh.k[buf][(kk / BS) * (KCH * 8) + (kk % BS) * 8 + half * BS * 8];
    f32x16_t sacc = {};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint4 a = *reinterpret_cast<const uint4*>(krow + st * 2 * BS * 8);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qb[st],
                                                     sacc, 0, 0, 0);
    }
    // ---- mask, online softmax -----------------------------------------------------------
    float sv[16];
    const bool need_mask = (kb + 32 > ctx) || (causal && kb + 31 > pos_first);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = sacc[r];
      if (need_mask) {
        const int kr = kb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (kr >= ctx || (causal && kr > qpos)) x = kNegInf;
      }
      sv[r] = x;
    }
    float mt = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sv[r]);
    mt = pair_max(mt) * qk_scale;        // scores are scaled by qk_scale > 0 below
    const float mn = fmaxf(m, mt);
    const float mref = (mn == kNegInf) ? 0.f : mn;
    if (__ballot(mn != m)) {  // some row's maximum grew: rescale sums and outputs
      const float alpha = fast_exp2(m - mref);  // 0 while m = -inf
      lsum *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] *= alpha;
        o1[r] *= alpha;
      }
      m = mn;
    }
    // p = 2^(s * qk_scale - m), rounded to bf16 once: the P.V operand; the running sum
    // adds those same rounded values (a dot with (1, 1)), so the normaliser matches.
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      pk[i] = pack_bf16x2(fast_exp2(__builtin_fmaf(sv[2 * i], qk_scale, -mref)),
                          fast_exp2(__builtin_fmaf(sv[2 * i + 1], qk_scale, -mref)));
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ps = dot2(pk[i], 0x3F803F80u, ps);
    lsum += ps;

    // ---- O^T += V^T . P^T ---------------------------------------------------------------
    // Element e (0..7) of lane half h's B operand for k-step ks is the score of key
    // 16 ks + (e < 4 ? 0 : 8) + 4 h + (e & 3) (the S^T accumulator order), so the V^T
    // operand reads the two 4-key runs at 16 ks + 4 h and 16 ks + 8 + 4 h.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 pb = make_uint4(pk[4 * ks + 0], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]);
      const int kr0 = 32 * hh + 16 * ks + 4 * half;  // first key (within the stage) of run 0
      const int pj = kr0 / BS;
      const int slot = kr0 % BS;  // runs at slot and slot + 8 stay inside one page
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint16_t* vr = &sh.v[buf][pj][32 * mb + j][slot];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + 8);
        const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
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
  };

  if (tid == 0) bad_sh = 0;
  if (n_stages > 0) {
    stage_load(0);
    stage_store(0, 0);
  }
  __syncthreads();
  for (int st = 0; st < n_stages; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < n_stages;
    if (more) stage_load(st + 1);
    const int k0 = st * kStage;
    compute_half(buf, k0, 0);
    if (k0 + 32 < kend) compute_half(buf, k0, 1);
    if (more) stage_store(st + 1, buf ^ 1);
    __syncthreads();
  }
  if (bad) bad_sh = 1;
  __syncthreads();

  // ---- normalise and store: lane holds dims 8*(r/4) + 4*half + (r%4) of query j ----------
  const float ltot = pair_sum(lsum);
  float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (bad_sh) inv = __builtin_nanf("");
  if (!qvalid) return;
  uint16_t* op = out + ((size_t)(qa + qi) * hq + head) * kHeadDim + 4 * half;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    uint2 v;
    v.x = pack_bf16x2(o0[4 * r4 + 0] * inv, o0[4 * r4 + 1] * inv);
    v.y = pack_bf16x2(o0[4 * r4 + 2] * inv, o0[4 * r4 + 3] * inv);
    *reinterpret_cast<uint2*>(op + 8 * r4) = v;
    v.x = pack_bf16x2(o1[4 * r4 + 0] * inv, o1[4 * r4 + 1] * inv);
    v.y = pack_bf16x2(o1[4 * r4 + 2] * inv, o1[4 * r4 + 3] * inv);
    *reinterpret_cast<uint2*>(op + 32 + 8 * r4) = v;
  }
}

}  // namespace

hipError_t launch_prefill(const LaunchGeom& geo, void* out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables, int max_blocks,
                          const int32_t* cu_q_lens, const int32_t* ctx_lens, int n_seqs,
                          int max_q_len, float scale, int causal, hipStream_t stream) {
  const int n_qtiles = (max_q_len + kQTile - 1) / kQTile;
  const dim3 grid((unsigned)((size_t)n_qtiles * n_seqs * geo.num_kv_heads));
  const dim3 block(kThreads);
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

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
// highest query positions see the most keys under the causal mask).  Small grids give a
// workgroup G key groups (each a copy of the four waves, taking every G-th stage, merged
// in LDS at the end), and the smallest split a tile's heads over two workgroups of two
// head-waves per group with four groups each.
//
// K/V stages: each key group copies 64 keys of K and V (the pages' own head slices)
// from the pools straight into LDS (global_load_lds: no staging registers, no LDS store
// instructions), once for all its head-waves, double-buffered: the copies of stage s+1 fly
// while the waves compute stage s.  K keeps the page's [8 pieces][bs][8] order (a wave's
// A-operand reads are then contiguous 512-byte runs).  V keeps the page's [64 dims][bs]
// rows with their 16-byte units XOR-swizzled by row, so the 16 rows one pass of a 16-byte
// read touches fall in distinct LDS banks.  Each half's S^T rows hold their keys in an
// order with bits 2 and 3 of the key swapped, which makes the 8 keys of each lane's V^T
// operand consecutive: one aligned 16-byte read.  After a copy lands, a wave zeroes the V
// values of keys past the context in the chunks it copied, so stale pool bytes (even NaN)
// never reach P.V.
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
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kQTile = 32;   // query positions per workgroup
constexpr int kStage = 64;   // keys per LDS stage
constexpr float kLazy = 8.f;  // log2 of the largest p the lazy rescale lets through
constexpr int kSlotFloats = kGroup * kQTile * kHeadDim;  // one partial output (fp32)
constexpr int kSlotRows = kGroup * kQTile;               // (max, sum) pairs of one partial

// Own value and the value of lane j ^ 32 (the two half-waves hold the same query's
// keys), in either order, from one v_permlane32_swap (it exchanges the upper half of its
// first operand with the lower half of its second): with both operands equal to x, the
// first is x[j] for j < 32 and x[j - 32] above, the second x[j + 32] below and x[j] above.
// Written as inline asm with both registers in/out: this compiler's builtin for the
// instruction hands back its first result for both.
__device__ __forceinline__ void pair_swap(float x, float& a, float& b) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  unsigned v = u;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(u), "+v"(v));  // pure: schedulable
  a = __builtin_bit_cast(float, u);
  b = __builtin_bit_cast(float, v);
}
// IEEE maximum (NaN-propagating): lowers to v_maximum3_f32 without the operand
// canonicalisation that fmaxf needs on MFMA results
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  pair_swap(x, a, b);
  return vmax(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  pair_swap(x, a, b);
  return a + b;  // same two operands in every lane of the pair
}

template <int BS>
struct PrefillLds {
  uint16_t k[2][kStage * kHeadDim];  // [buffer][page][8][bs][8]: the pages' own order
  uint16_t v[2][kStage * kHeadDim];  // [buffer][page][dim][bs], 16-byte units swizzled
};
// V rows in LDS: the 16-byte units (8 keys) of dim row r sit at unit position u ^ vswz(r),
// so the 16 rows one pass of a 16-byte read touches fall in distinct LDS banks.
template <int BS>
__device__ __forceinline__ int vswz(int row) {
  return BS == 16 ? (row >> 3) & 1 : (row >> 2) & 3;
}
// Wait until this wave's copies into LDS have landed (vector-memory count 0; the compiler
// does not count these copies itself), and keep memory accesses from moving above it.
__device__ __forceinline__ void wait_copies() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt free
  asm volatile("" ::: "memory");
}

template <int BS, int G, int HPW>
__global__ __launch_bounds__(64 * HPW * G) __attribute__((amdgpu_waves_per_eu(HPW == kGroup ? 3 : 2)))
void prefill_kernel(
    uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ ctx_lens, int n_seqs,
    int n_qtiles, int num_pages, int num_kv_heads, float qk_scale, int causal, int n_split,
    float* __restrict__ ws_o, float2* __restrict__ ws_ml) {
  using Lds = PrefillLds<BS>;
  constexpr int KCH = 8 * BS;  // 16-byte chunks of one page's K (or V) head slice
  constexpr int kGT = 64 * HPW;          // threads of one key group: a wave per query head
  constexpr int NHP = kGroup / HPW;      // workgroups sharing one tile, by query heads
  constexpr int NC = kStage * kHeadDim / 8 / kGT;  // 16-byte K (and V) chunks per thread
  static_assert(NC * kGT * 8 == kStage * kHeadDim && KCH % 64 == 0, "staging");
  __shared__ __attribute__((aligned(16))) Lds sh_all[G];

  // Work order: tiles longest first (highest query positions see the most keys), the
  // sequences of one tile level rotated by the level.  The hardware hands workgroups to
  // the XCDs (bid mod 8) and, inside one, to its shader engines in turn; without the
  // rotation a sequence would land on the same engine at every level and the engines'
  // loads would differ by the sequences' lengths.
  // With HPW < 4 the query heads of a tile are shared out over NHP workgroups (Hkv apart,
  // so on one XCD); with n_split > 1 the tile's keys are also cut into n_split pieces
  // (NHP * Hkv workgroups apart).  The KV head stays bid mod Hkv.
  const int bid = blockIdx.x;
  const int g = bid % num_kv_heads;
  const int hp = (bid / num_kv_heads) % NHP;
  const int piece = (bid / (num_kv_heads * NHP)) % n_split;
  const int tb = bid / (num_kv_heads * NHP * n_split);  // tile-level position
  const int level = tb / n_seqs;
  const int s = (tb % n_seqs + level) % n_seqs;
  const int tile = n_qtiles - 1 - level;
  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x / kGT);  // key group
  Lds& sh = sh_all[grp];
  const int tid = threadIdx.x % kGT;  // thread within the group
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;    // query column of this lane
  const int half = lane >> 5;
  const int hq = num_kv_heads * kGroup;
  const int hw = hp * HPW + w;  // this wave's query head within the KV head's group
  const int head = g * kGroup + hw;

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
  const int klim = causal ? min(ctx, qpos + 1) : ctx;        // this lane's row sees keys < klim
  const int n_all = (kend + kStage - 1) / kStage;       // stages of the whole tile
  // A row that sees few keys gets its output from a few large weights, and one bf16
  // term per probability (8 significant bits) can then move it by 2^-8 of the spread of
  // those keys' V values.  Tiles holding a row that sees fewer than 64 keys therefore
  // feed P.V two bf16 terms per probability (hi = bf16(p), lo = bf16(p - hi): 16 bits).
  const bool precise = (causal ? min(ctx, pos_first + 1) : ctx) < kStage;
  const int st0 = piece * n_all / n_split;              // this piece: stages st0 .. +n_stages
  const int n_stages = (piece + 1) * n_all / n_split - st0;
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

  // ---- staging: 16-byte chunks c of a stage, copied from the pools straight into LDS ---
  // chunk c of a stage: page c / KCH, 16-byte piece c % KCH of that page's head slice.
  // A page slice is KCH >= 128 chunks, so each wave's 64 chunks of either kind in one
  // instruction lie in one page: block-table entries and page addresses are wave-uniform
  // (scalar registers), and a lane only adds its byte offset within the page.
  const size_t page_bytes = page_stride * sizeof(uint16_t);
  const char* k_base = reinterpret_cast<const char*>(k_head);
  const char* v_base = reinterpret_cast<const char*>(v_head);
  // Block-table entries of the wave's pages of stage st (one per chunk instruction), pages
  // past the last needed block repeating it.
  auto stage_pids = [&](int st, int (&pid)[NC]) __attribute__((always_inline)) {
    const int blk0 = st * (kStage / BS);
#pragma unroll
    for (int i = 0; i < NC; ++i)
      pid[i] = bt[__builtin_amdgcn_readfirstlane(min(blk0 + (64 * w + kGT * i) / KCH, last_blk))];
  };
  // Instruction i of wave w fills LDS chunks c0 .. c0 + 63, c0 = 64 (w + HPW i), of the K
  // and of the V buffer (lane l writes chunk c0 + l: the copy's LDS address is the
  // instruction's base plus 16 bytes per lane).  K chunks keep the page's order; lane l of
  // a V instruction fetches the page's unit that belongs at its swizzled position.
  // Returns the bits of the instructions whose page id was out of range (page 0 was
  // read instead; stage_fix overwrites those chunks).
  auto stage_dma = [&](int buf, const int (&pid)[NC]) __attribute__((always_inline)) -> int {
    int bad = 0;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      int pg = __builtin_amdgcn_readfirstlane(pid[i]);
      if ((unsigned)pg >= (unsigned)num_pages) {
        bad |= 1 << i;
        pg = 0;
      }
      const int c0 = 64 * (w + HPW * i);
      const int within = c0 % KCH + lane;  // chunk within the page slice
      const int row = within / (BS / 8);
      const int u = (within % (BS / 8)) ^ vswz<BS>(row);
      const size_t pgo = (size_t)pg * page_bytes;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(k_base + pgo + (size_t)within * 16),
          (__attribute__((address_space(3))) void*)&sh.k[buf][c0 * 8], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(v_base + pgo +
                                                           (size_t)(row * (BS / 8) + u) * 16),
          (__attribute__((address_space(3))) void*)&sh.v[buf][c0 * 8], 16, 0, 0);
    }
    return bad;
  };
  // After this wave's copies of a stage have landed: its chunks from an out-of-range page
  // become K = NaN, V = 0, and V values of keys at or past the context end become 0 (stale
  // pool bytes, even NaN, must not meet a zero probability in P.V).  Each lane touches only
  // the chunks it copied itself, so the stage barrier that follows publishes both.
  auto stage_fix = [&](int st, int buf, int bad) __attribute__((always_inline)) {
    const int k0 = st * kStage;
    const bool tail = k0 + kStage > ctx;
    if (__builtin_expect(bad == 0 && !tail, 1)) return;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = 64 * (w + HPW * i) + lane;
      u32x4_t* kd = reinterpret_cast<u32x4_t*>(&sh.k[buf][c * 8]);
      u32x4_t* vd = reinterpret_cast<u32x4_t*>(&sh.v[buf][c * 8]);
      if (bad & (1 << i)) {
        *kd = u32x4_t{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u};
        *vd = u32x4_t{0u, 0u, 0u, 0u};
      } else if (tail) {
        const int pj = c / KCH;
        const int within = c % KCH;
        const int row = within / (BS / 8);
        const int u = (within % (BS / 8)) ^ vswz<BS>(row);
        const int key0 = k0 + pj * BS + 8 * u;
        if (key0 + 8 > ctx) {
          u32x4_t vv = *vd;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (key0 + e >= ctx) vv[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          *vd = vv;
        }
      }
    }
  };

  // This lane's query row: reference maximum m (scaled), m + kLazy, the FMA addend -m (0
  // while m is -inf, so masked scores give 2^-inf = 0), and the running sum.
  float m = kNegInf, mthr = kNegInf, negm = 0.f, lsum = 0.f;  // mthr: raw-score units
  const float inv_scale = 1.f / qk_scale;
  const int lim_lane = klim - 8 * half;  // key offsets from a half's base below this are visible
  f32x16_t o0 = {}, o1 = {};

  // A stage is two 32-key halves.  Per half: S^T = K . Q^T (4 MFMAs), the online-softmax
  // update (VALU), O^T += V^T . P^T (4 MFMAs).  The stage issues both halves' S^T products
  // first, so the softmax of one half runs on the VALU while the matrix core works on the
  // other's products; reductions are trees rather than chains.
  // K operands of one half (4 x 16 bytes: pieces 2 st + half of the lane's key row)
  struct KOps {
    u32x4_t a[4];
  };
  // Row j of a half's S^T holds key sig(j): bits 2 and 3 of j trade places.  The P^T operand
  // then carries keys 16 ks + 8 h .. 16 ks + 8 h + 7 in lane half h, eight keys in a row, so
  // the V^T operand is one 16-byte unit.
  const int sig_j = (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
  auto read_k = [&](int buf, int hh, KOps& ko) __attribute__((always_inline)) {
    const int kk = 32 * hh + sig_j;  // key within the stage held as A row by this lane
    const uint16_t* krow =
        &sh.k[buf][(kk / BS) * (KCH * 8) + (kk % BS) * 8 + half * BS * 8];
#pragma unroll
    for (int st = 0; st < 4; ++st) ko.a[st] = *reinterpret_cast<const u32x4_t*>(krow + st * 2 * BS * 8);
  };
  auto qk = [&](const KOps& ko) __attribute__((always_inline)) -> f32x16_t {
    f32x16_t sacc = {};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ko.a[st]),
                                                     qb[st], sacc, 0, 0, 0);
    return sacc;
  };
  // mask, online-softmax update; returns p (bf16 pairs) in the S^T accumulator order, and
  // with `precise` also the pairs of the remainders p - hi in pl
  auto softmax = [&](const f32x16_t& sacc, int kb, uint32_t (&pk)[8], uint32_t (&pl)[8],
                     auto precise_tag) __attribute__((always_inline)) {
    constexpr bool PRECISE = decltype(precise_tag)::value;
    float sv[16];
    if ((kb + 32 > ctx) || (causal && kb + 31 > pos_first)) {  // the half crosses a limit
      // element r is row 8 (r / 4) + 4 half + r % 4 of S^T, which holds key
      // kb + 16 (r / 8) + 8 half + 4 ((r / 4) % 2) + r % 4; visible while below klim
      const int lim = lim_lane - kb;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sv[r] = (16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3)) < lim ? sacc[r] : kNegInf;
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[r] = sacc[r];
    }
    const float t0 = vmax3(sv[0], sv[1], sv[2]), t1 = vmax3(sv[3], sv[4], sv[5]);
    const float t2 = vmax3(sv[6], sv[7], sv[8]), t3 = vmax3(sv[9], sv[10], sv[11]);
    const float t4 = vmax3(sv[12], sv[13], sv[14]);
    float mt = vmax3(vmax3(t0, t1, t2), vmax(t3, t4), sv[15]);
    mt = pair_max(mt);  // raw scores; scaled by qk_scale > 0 below
    // Lazy rescale: the running maximum m is only a reference point, any value works as
    // long as sums and outputs use the same one.  It is moved (and sums and outputs
    // rescaled) only when a row's new maximum exceeds it by more than 2^kLazy, so p stays
    // <= 2^kLazy and the rescale runs about once per row instead of nearly every tile.
    if (__ballot(mt > mthr)) {
      const float mn = vmax(m, mt * qk_scale);
      const float alpha = m == kNegInf ? 0.f : fast_exp2(m - mn);
      if (__ballot(m != kNegInf)) {  // rows still at -inf hold o = 0, l = 0: nothing to scale
        lsum *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          o0[r] *= alpha;
          o1[r] *= alpha;
        }
      }
      m = mn;
      mthr = (m + kLazy) * inv_scale;
      negm = m == kNegInf ? 0.f : -m;
    }
    // p = 2^(s * qk_scale - m), rounded to bf16 once: the P.V operand; the running sum
    // adds those same rounded values (a dot with (1, 1)), so the normaliser matches.
    if constexpr (PRECISE) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p0 = fast_exp2(__builtin_fmaf(sv[2 * i], qk_scale, negm));
        const float p1 = fast_exp2(__builtin_fmaf(sv[2 * i + 1], qk_scale, negm));
        pk[i] = pack_bf16x2(p0, p1);
        pl[i] = pack_bf16x2(p0 - bf_lo(pk[i]), p1 - bf_hi(pk[i]));
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lsum = dot2(pk[i], 0x3F803F80u, lsum);
        lsum = dot2(pl[i], 0x3F803F80u, lsum);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pk[i] = pack_bf16x2(fast_exp2(__builtin_fmaf(sv[2 * i], qk_scale, negm)),
                            fast_exp2(__builtin_fmaf(sv[2 * i + 1], qk_scale, negm)));
#pragma unroll
      for (int i = 0; i < 8; ++i) lsum = dot2(pk[i], 0x3F803F80u, lsum);
    }
  };
  // O^T += V^T . P^T.  Element e (0..7) of lane half h's B operand for k-step ks is S^T
  // row 16 ks + 8 (e / 4) + 4 h + e % 4 (the accumulator order), which holds key
  // 16 ks + 8 h + e (the rows' key order above), so the V^T operand is the 8 keys from
  // 16 ks + 8 h: one 16-byte unit of a V row.
  struct VOps {
    u32x4_t a[2][2];  // [ks][mb]
  };
  auto read_v = [&](int buf, int hh, VOps& vo) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kg = 32 * hh + 16 * ks + 8 * half;  // first of the lane's 8 keys (in the stage)
      const int pj = kg / BS;
      const int u = (kg % BS) / 8;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * mb + j;
        vo.a[ks][mb] = *reinterpret_cast<const u32x4_t*>(
            &sh.v[buf][(pj * kHeadDim + row) * BS + 8 * (u ^ vswz<BS>(row))]);
      }
    }
  };
  auto pv = [&](const VOps& vo, const uint32_t (&pk)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t pb = {pk[4 * ks + 0], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vo.a[ks][0]),
                                                   __builtin_bit_cast(bf16x8_t, pb), o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vo.a[ks][1]),
                                                   __builtin_bit_cast(bf16x8_t, pb), o1, 0, 0, 0);
    }
  };
  // The second half's softmax and P.V are skipped when it lies wholly past kend; its S^T
  // products are issued with the first half's, so they are in flight during the first
  // half's softmax.  All K and V operands of the stage are read from LDS up front (with the
  // copies going straight to LDS there is room for them at three waves per SIMD).
  auto compute_stage_fast = [&](int buf, int k0) __attribute__((always_inline)) {
    KOps k0o, k1o;
    read_k(buf, 0, k0o);
    read_k(buf, 1, k1o);
    uint32_t p0[8], p1[8], unused[8];
    const f32x16_t s0 = qk(k0o);
    const f32x16_t s1 = qk(k1o);
    VOps v0o, v1o;
    read_v(buf, 0, v0o);
    read_v(buf, 1, v1o);
    softmax(s0, k0, p0, unused, std::false_type{});
    pv(v0o, p0);
    if (__builtin_expect(k0 + 32 < kend, 1)) {  // else masked whole: nothing to add
      softmax(s1, k0 + 32, p1, unused, std::false_type{});
      pv(v1o, p1);
    }
  };
  // The same for a tile with rows that see few keys: the halves one after the other (so
  // the remainders' registers fit where the second half's scores sat), P.V over the hi
  // terms, then over the lo terms.
  auto compute_stage_precise = [&](int buf, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 0 || k0 + 32 < kend) {
        KOps ko;
        read_k(buf, hh, ko);
        const f32x16_t sh_ = qk(ko);
        VOps vo;
        read_v(buf, hh, vo);
        uint32_t ph[8], pl[8];
        softmax(sh_, k0 + 32 * hh, ph, pl, std::true_type{});
        pv(vo, ph);
        pv(vo, pl);
      }
    }
  };

  // Key groups: group grp takes the piece's stages grp, grp + G, grp + 2G, ... (round u
  // holds stage grp + G u of every group); every group runs the same number of rounds, so
  // the workgroup barriers match, and a round past the group's last stage copies and
  // computes nothing.
  const int n_u = (n_stages + G - 1) / G;
  auto stage_of = [&](int u) __attribute__((always_inline)) { return st0 + grp + G * u; };
  auto live_of = [&](int u) __attribute__((always_inline)) { return grp + G * u < n_stages; };
  // Both paths stage round by round: a wave's copies of a round go straight into LDS, the
  // wave waits for them (wait_copies), patches its own chunks (stage_fix), and the
  // workgroup barrier publishes the round.  No copy is issued for a round past the
  // group's last, and none is in flight when a wave leaves its loop.
  if (__builtin_expect(precise, 0)) {
    // A tile with rows that see few keys has at most two stages (causal: its keys end
    // within 32 of its first row, which sits below 63; otherwise the context is shorter
    // than a stage): staged one at a time, without the pipeline.
    for (int u = 0; u < n_u; ++u) {
      int bad = 0;
      if (live_of(u)) {
        int pid_s[NC];
        stage_pids(stage_of(u), pid_s);
        bad = stage_dma(u & 1, pid_s);
      }
      wait_copies();
      if (live_of(u)) stage_fix(stage_of(u), u & 1, bad);
      __syncthreads();
      if (live_of(u)) compute_stage_precise(u & 1, stage_of(u) * kStage);
    }
  } else {
    // Stage pipeline (in rounds).  Round u computes the group's stage of round u from
    // buffer u % 2 while the copies of round u + 1 fly into the other buffer (left by round
    // u - 1 before the last barrier); block-table entries run a round further ahead.
    int pid_n[NC] = {};  // entries of the next round to copy
    {
      int pid0[NC] = {};
      if (n_u > 0) stage_pids(stage_of(0), pid0);
      // An explicit use of q before the first copy: the compiler (which does not count
      // the copies) waits for q here, while the first block-table entries are in flight,
      // and knows q has arrived on every path into the loop.
      asm volatile("" ::"v"(qb[0]), "v"(qb[1]), "v"(qb[2]), "v"(qb[3]));
      int bad0 = 0;
      if (live_of(0)) bad0 = stage_dma(0, pid0);
      if (n_u > 0) stage_pids(stage_of(1), pid_n);
      wait_copies();
      if (live_of(0)) stage_fix(stage_of(0), 0, bad0);
    }
    __syncthreads();
    for (int u = 0; u < n_u; ++u) {
      int bad_n = 0;
      if (live_of(u + 1)) bad_n = stage_dma((u + 1) & 1, pid_n);
      stage_pids(stage_of(u + 2), pid_n);
      if (live_of(u)) compute_stage_fast(u & 1, stage_of(u) * kStage);
      wait_copies();
      if (live_of(u + 1)) stage_fix(stage_of(u + 1), (u + 1) & 1, bad_n);
      __syncthreads();
    }
  }

  if constexpr (G > 1) {
    // Merge of the key groups through LDS (the stage buffers are free once every group
    // has finished): groups 1 .. G-1 leave their reference maxima, lane sums and output
    // accumulators; group 0 combines them, M = max m_g, weights 2^(m_g - M) (0 for a
    // group that saw no key of the row), and goes on with the result alone.
    constexpr int kF = 34;  // floats per lane: o0, o1, m, lsum
    static_assert((G - 1) * HPW * kF * 64 * sizeof(float) <= sizeof(sh_all), "merge space");
    float* mb = reinterpret_cast<float*>(sh_all);
    __syncthreads();
    if (grp > 0) {
      float* dst = mb + ((size_t)((grp - 1) * HPW + w) * kF) * 64 + lane;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dst[r * 64] = o0[r];
        dst[(16 + r) * 64] = o1[r];
      }
      dst[32 * 64] = m;
      dst[33 * 64] = lsum;
    }
    __syncthreads();
    if (grp > 0) return;
    float mg[G - 1], M = m;
#pragma unroll
    for (int k = 1; k < G; ++k) {
      mg[k - 1] = mb[((size_t)((k - 1) * HPW + w) * kF + 32) * 64 + lane];
      M = vmax(M, mg[k - 1]);
    }
    const float f0 = m == kNegInf ? 0.f : fast_exp2(m - M);
    lsum *= f0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      o0[r] *= f0;
      o1[r] *= f0;
    }
#pragma unroll
    for (int k = 1; k < G; ++k) {
      const float* srcp = mb + ((size_t)((k - 1) * HPW + w) * kF) * 64 + lane;
      const float f = mg[k - 1] == kNegInf ? 0.f : fast_exp2(mg[k - 1] - M);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o0[r] = __builtin_fmaf(f, srcp[r * 64], o0[r]);
        o1[r] = __builtin_fmaf(f, srcp[(16 + r) * 64], o1[r]);
      }
      lsum = __builtin_fmaf(f, srcp[33 * 64], lsum);
    }
    m = M;
  }

  if (n_split > 1) {
    // a piece: fp32 partial (reference maximum, sum, unnormalised output) for the merge,
    // slot (item, piece) with item = (tile * n_seqs + s) * Hkv + g, in lane order: wave w's
    // accumulator chunk r (o0 then o1, 4 floats) of lane l at float (hw * 8 + r) * 256 + 4 l
    // (hw: the wave's query head within the KV head's group),
    // so every store (and the merge's load) moves one contiguous kilobyte
    const float ltot = pair_sum(lsum);
    const size_t slot = ((size_t)(tile * n_seqs + s) * num_kv_heads + g) * n_split + piece;
    float* po = ws_o + slot * kSlotFloats + hw * 8 * 256 + 4 * lane;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      *reinterpret_cast<f32x4_t*>(po + r4 * 256) =
          f32x4_t{o0[4 * r4], o0[4 * r4 + 1], o0[4 * r4 + 2], o0[4 * r4 + 3]};
      *reinterpret_cast<f32x4_t*>(po + (4 + r4) * 256) =
          f32x4_t{o1[4 * r4], o1[4 * r4 + 1], o1[4 * r4 + 2], o1[4 * r4 + 3]};
    }
    if (half == 0) ws_ml[slot * kSlotRows + hw * kQTile + j] = make_float2(m, ltot);
    return;
  }

  // ---- normalise and store: lane holds dims 8*(r/4) + 4*half + (r%4) of query j ----------
  const float ltot = pair_sum(lsum);
  const float inv = ltot == 0.f ? 0.f : 1.f / ltot;  // a NaN sum stays NaN
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

// Merge of a split tile: one wave per (item, head), item = (tile * n_seqs + s) * Hkv + g;
// lane (j, half) holds the same dims as the split kernel wrote (its lane-ordered chunks).  The pieces combine by log-sum-exp in
// piece order: M = max m_p, out = sum 2^(m_p - M) o_p / sum 2^(m_p - M) l_p; all pieces'
// loads are issued before any is used.  A NaN piece (a row that saw an out-of-range
// page) stays NaN.
template <int NS>
__global__ __launch_bounds__(64) void prefill_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_o, const float2* __restrict__ ws_ml,
    const int32_t* __restrict__ cu_q_lens, int n_seqs, int num_kv_heads) {
  const int item = blockIdx.x / kGroup;  // one single-wave workgroup per (item, head)
  const int w = blockIdx.x % kGroup;
  const int g = item % num_kv_heads;
  const int s = (item / num_kv_heads) % n_seqs;
  const int tile = item / (num_kv_heads * n_seqs);
  const int lane = threadIdx.x;
  const int j = lane & 31;
  const int half = lane >> 5;
  const size_t slot0 = (size_t)item * NS;
  float2 ml[NS];
  f32x4_t x[NS][8];
#pragma unroll
  for (int p = 0; p < NS; ++p) {
    ml[p] = ws_ml[(slot0 + p) * kSlotRows + w * kQTile + j];
    const float* po = ws_o + (slot0 + p) * kSlotFloats + w * 8 * 256 + 4 * lane;
#pragma unroll
    for (int r = 0; r < 8; ++r) x[p][r] = *reinterpret_cast<const f32x4_t*>(po + r * 256);
  }
  const int qa = cu_q_lens[s];
  const int qlen = cu_q_lens[s + 1] - qa;
  const int qi = tile * kQTile + j;
  if (qi >= qlen) return;
  float mx = kNegInf;
#pragma unroll
  for (int p = 0; p < NS; ++p) mx = vmax(mx, ml[p].x);
  float acc[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) acc[e] = 0.f;
  float lt = 0.f;
  if (mx != kNegInf) {
#pragma unroll
    for (int p = 0; p < NS; ++p) {
      const float wgt = fast_exp2(ml[p].x - mx);  // 0 for a piece without visible keys
      lt += wgt * ml[p].y;
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * r + e] += wgt * x[p][r][e];
    }
  }
  const float inv = lt == 0.f ? 0.f : 1.f / lt;
  const int hq = num_kv_heads * kGroup;
  // acc[4 r + e] is dim 8 (r % 4) + 4 half + e, + 32 for r >= 4 (the o0 / o1 order)
  uint16_t* op = out + ((size_t)(qa + qi) * hq + g * kGroup + w) * kHeadDim + 4 * half;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    uint2 v;
    v.x = pack_bf16x2(acc[4 * r + 0] * inv, acc[4 * r + 1] * inv);
    v.y = pack_bf16x2(acc[4 * r + 2] * inv, acc[4 * r + 3] * inv);
    *reinterpret_cast<uint2*>(op + (r < 4 ? 8 * r : 32 + 8 * (r - 4))) = v;
  }
}

}  // namespace

PrefillPlan plan_prefill(int n_seqs, int max_q_len, int max_ctx_len, int num_kv_heads,
                         int kv_splits, int compute_units) {
  PrefillPlan p{};
  const int64_t items = (int64_t)((max_q_len + kQTile - 1) / kQTile) * n_seqs * num_kv_heads;
  const int64_t stages = std::max<int64_t>(1, ((int64_t)max_ctx_len + kStage - 1) / kStage);
  const int64_t cus = std::max(compute_units, 1);
  p.items = items;
  // A grid smaller than the chip gives each tile two key groups (eight waves), halving the
  // serial stage chain of its workgroup; at most half the chip, each tile goes to two
  // workgroups of two query heads with four key groups each (eight waves again, a quarter
  // of the chain).  A larger grid keeps three four-wave workgroups per compute unit.
  if (items > 0 && 2 * items <= cus) {
    p.groups = 4;
    p.heads = 2;
  } else {
    p.groups = items > 0 && items < cus ? 2 : 1;
    p.heads = kGroup;
  }
  const int64_t wgs = items * (kGroup / p.heads);  // workgroups per key piece
  int64_t split = kv_splits;
  if (split == 0) {  // at most 8 pieces, never more than the stages
    // one-group workgroups: enough for two per compute unit; several groups: enough for
    // half the compute units (the pieces' merge costs more than the idle units)
    const int64_t want = p.groups == 1 ? 2 * cus : cus / 2;
    split = wgs > 0 && wgs < want ? (want + wgs - 1) / wgs : 1;
    split = std::min<int64_t>(std::min<int64_t>(split, kPrefillMaxSplit), stages);
  }
  p.split = (int)std::max<int64_t>(split, 1);
  if (p.split > 1)
    p.ws_bytes = (size_t)items * p.split * (kSlotFloats * sizeof(float) + kSlotRows * sizeof(float2));
  return p;
}

hipError_t launch_prefill(const LaunchGeom& geo, const PrefillPlan& plan, void* out, const void* q,
                          const void* k_pool, const void* v_pool, const int32_t* block_tables,
                          int max_blocks, const int32_t* cu_q_lens, const int32_t* ctx_lens,
                          int n_seqs, int max_q_len, float scale, int causal, void* workspace,
                          hipStream_t stream) {
  const int n_qtiles = (max_q_len + kQTile - 1) / kQTile;
  const int ns = plan.split;
  const dim3 grid((unsigned)(plan.items * (kGroup / plan.heads) * ns));
  const dim3 block(64 * plan.heads * plan.groups);
  const float qk_scale = scale * kLog2e;
  auto* o = static_cast<uint16_t*>(out);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kp = static_cast<const uint16_t*>(k_pool);
  auto* vp = static_cast<const uint16_t*>(v_pool);
  float* ws_o = nullptr;
  float2* ws_ml = nullptr;
  if (ns > 1) {
    ws_o = static_cast<float*>(workspace);
    ws_ml = reinterpret_cast<float2*>(ws_o + (size_t)plan.items * ns * kSlotFloats);
  }
#define PA_PREFILL_LAUNCH(B, NG, NH)                                                          \
  hipLaunchKernelGGL((prefill_kernel<B, NG, NH>), grid, block, 0, stream, o, qq, kp, vp,         \
                     block_tables, max_blocks, cu_q_lens, ctx_lens, n_seqs, n_qtiles,            \
                     geo.num_pages, geo.num_kv_heads, qk_scale, causal, ns, ws_o, ws_ml)
  if (geo.block_size == 16) {
    if (plan.groups == 4) PA_PREFILL_LAUNCH(16, 4, 2);
    else if (plan.groups == 2) PA_PREFILL_LAUNCH(16, 2, 4);
    else PA_PREFILL_LAUNCH(16, 1, 4);
  } else {
    if (plan.groups == 4) PA_PREFILL_LAUNCH(32, 4, 2);
    else if (plan.groups == 2) PA_PREFILL_LAUNCH(32, 2, 4);
    else PA_PREFILL_LAUNCH(32, 1, 4);
  }
#undef PA_PREFILL_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns == 1) return e;
  const dim3 mgrid((unsigned)(plan.items * kGroup));
  switch (ns) {
#define PA_MERGE_CASE(N)                                                                    \
  case N:                                                                                   \
    hipLaunchKernelGGL(prefill_merge_kernel<N>, mgrid, dim3(64), 0, stream, o, ws_o, ws_ml, \
                       cu_q_lens, n_seqs, geo.num_kv_heads);                                \
    break;
    PA_MERGE_CASE(2)
    PA_MERGE_CASE(3)
    PA_MERGE_CASE(4)
    PA_MERGE_CASE(5)
    PA_MERGE_CASE(6)
    PA_MERGE_CASE(7)
    PA_MERGE_CASE(8)
#undef PA_MERGE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa

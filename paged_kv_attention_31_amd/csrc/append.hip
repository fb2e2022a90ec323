// kv_append and rope_kv_append: write the new tokens' K and V rows into their pages,
// optionally turning Q and K by rotary position encoding on the way.
//
// A token's K/V joins the page cache before the token attends
// ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §推理流程：从Prefill到Decode); page and
// slot come from the block table (same page, §PagedAttention：从操作系统借来的智慧).  The
// attention sub-layer turns Q and K by the token's position before attention (same
// page, §Llama 3.2 1B架构拆解); fusing that rotation into the append reads and writes
// each new row once.
//
// One workgroup of 256 threads takes a block of 8 rows (tokens): normally 8 positions
// 8j .. 8j+7 of one sequence (see kFastSeqs).  Per row it finds the token, position,
// page and slot once (8 lanes), then:
//   K  (page layout [Hkv][8][bs][8]): a thread moves one (row, head, piece pair): the
//      16-byte pieces k and k + 4 hold dims 8k..8k+7 and 32+8k..39+8k, the two halves of
//      the rotation pairs, so a rotated piece pair never leaves the thread;
//   V  (page layout [Hkv][64][bs]): the 8 rows are staged through LDS and written per
//      (head, dim) page row; when the 8 tokens fill slots 8j..8j+7 of one page (a
//      prefill or prompt chunk) each page row gets one 16-byte store, otherwise one
//      2-byte store per token (decode: one token per sequence);
//   Q  (rope only): each thread rotates piece pairs of the rows' query heads in place
//      or into q_out.
// Rotation: pair i is (x[i], x[i + 32]), angle pos * f_i with f_i = theta^(-2i/64) or a
// caller-given table; the angle is formed and reduced modulo 2 pi in fp64, its cosine
// and sine rounded to fp32, the rotation done in fp32 and rounded once to bf16.
// The new rows of K, V and Q are read once, with nontemporal loads.
#include "common.h"
#include "launch.h"

namespace pa {

namespace {

constexpr int kRows = 8;  // tokens per workgroup
constexpr double kTwoPi = 6.283185307179586476925286766559;

// sequence s with cu[s] <= t < cu[s+1] (cu ascending, cu[0] = 0)
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu, int n_seqs, int t) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Rotate eight pairs: a holds dims i..i+7, b dims i+32..i+39 (bf16 bit pairs).
__device__ __forceinline__ void rotate8(u32x4_t& a, u32x4_t& b, const float* c, const float* s) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a0 = bf_lo(a[w]), a1 = bf_hi(a[w]), b0 = bf_lo(b[w]), b1 = bf_hi(b[w]);
    const float c0 = c[2 * w], c1 = c[2 * w + 1], s0 = s[2 * w], s1 = s[2 * w + 1];
    a[w] = pack_bf16x2(__builtin_fmaf(a0, c0, -b0 * s0), __builtin_fmaf(a1, c1, -b1 * s1));
    b[w] = pack_bf16x2(__builtin_fmaf(b0, c0, a0 * s0), __builtin_fmaf(b1, c1, a1 * s1));
  }
}

// Up to this many sequences (one thread per cumulative length, n_seqs + 1 of them), the
// lengths are read into LDS in one round trip and the workgroups take position-aligned
// blocks: block j of sequence s holds its new tokens at positions 8j .. 8j+7, so a full
// block fills 8 consecutive slots of one page and its V page rows are written 16 bytes at
// a time.  Each sequence's blocks are numbered from a multiple of block_size / 8 (padding
// blocks do nothing), so the blocks of one page are consecutive numbers.  With more
// sequences the blocks are 8 consecutive packed rows and each row searches the device
// array (one dependent load per halving).
constexpr int kFastSeqs = 255;
// Q piece pairs each thread holds at once (all of them for up to 32 query heads).
constexpr int kQBatch = 4;

template <int BS, bool ROPE>
__global__ __launch_bounds__(256) void append_kernel(
    const uint16_t* q_in, uint16_t* q_out,  // rope only; q_out may be q_in (in place)
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ cu_new_lens, const int32_t* __restrict__ ctx_lens, int n_seqs,
    int n_tokens, int num_q_heads, int num_kv_heads, int num_pages, double log2_theta,
    const float* __restrict__ inv_freq) {
  constexpr int GS = BS / kRows;  // blocks per page
  __shared__ int cu_sh[kFastSeqs + 1], ctx_sh[kFastSeqs], nb_sh[256], wsum_sh[4], cnt_sh[4];
  __shared__ int tok_sh[kRows], page_sh[kRows], slot_sh[kRows], pos_sh[kRows];
  __shared__ float cos_sh[ROPE ? kRows : 1][kHeadDim / 2], sin_sh[ROPE ? kRows : 1][kHeadDim / 2];
  extern __shared__ __attribute__((aligned(16))) uint16_t v_sh[];  // [kRows][Hkv][64]
  const int tid = threadIdx.x;
  // The GS blocks of one page write parts of the same V page rows; they run on one XCD
  // (bid mod 8), so those partial rows meet in one L2 before they reach HBM: logical
  // block GS m + j takes bid 8 (GS (m / 8) + j) + m mod 8.
  const int xcd = blockIdx.x % 8, kk = blockIdx.x / 8;
  const int blk = GS * (8 * (kk / GS) + xcd) + kk % GS;
  const int hd = num_kv_heads * kHeadDim;  // elements of one token's K (or V) row
  const int qd = num_q_heads * kHeadDim;
  const bool fast = n_seqs <= kFastSeqs;

  // ---- rows of this block: token index (or -1), sequence, position ----------------------
  int my_s = 0, my_tok = -1, my_pos = 0;  // lanes 0..7: row tid
  if (fast) {
    if (tid <= n_seqs) cu_sh[tid] = cu_new_lens[tid];
    if (tid < n_seqs) ctx_sh[tid] = ctx_lens[tid];
    __syncthreads();
    // blocks of sequence tid: positions [first_pos, ctx) in aligned groups of GS blocks
    int nb = 0;
    if (tid < n_seqs) {
      const int n_s = cu_sh[tid + 1] - cu_sh[tid];
      const int fp = ctx_sh[tid] - n_s;
      if (n_s > 0) {
        const int j0 = (fp >= 0 ? fp / (8 * GS) : -((-fp + 8 * GS - 1) / (8 * GS))) * GS;
        const int j1 = (ctx_sh[tid] + 8 * GS - 1) / (8 * GS) * GS;
        nb = max(j1 - j0, 0);
      }
    }
    // inclusive scan of the block counts: inside each wave by lane shuffles, then the
    // totals of the lower waves added
    const int wv = tid >> 6;
    int inc = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(inc, off, 64);
      if ((tid & 63) >= off) inc += y;
    }
    if ((tid & 63) == 63) wsum_sh[wv] = inc;
    __syncthreads();
    for (int k = 0; k < wv; ++k) inc += wsum_sh[k];
    if (blk >= wsum_sh[0] + wsum_sh[1] + wsum_sh[2] + wsum_sh[3]) return;  // uniform
    nb_sh[tid] = inc;
    // the block's sequence is the first whose inclusive count exceeds blk: the number of
    // sequences whose count does not (the counts never decrease)
    const unsigned long long le = __ballot(tid < n_seqs && inc <= blk);
    if ((tid & 63) == 0) cnt_sh[wv] = __popcll(le);
    __syncthreads();
    const int s = cnt_sh[0] + cnt_sh[1] + cnt_sh[2] + cnt_sh[3];
    const int first = cu_sh[s], n_s = cu_sh[s + 1] - first, fp = ctx_sh[s] - n_s;
    const int j0 = (fp >= 0 ? fp / (8 * GS) : -((-fp + 8 * GS - 1) / (8 * GS))) * GS;
    const int j = j0 + blk - (s > 0 ? nb_sh[s - 1] : 0);
    if (tid < kRows) {
      const int p = 8 * j + tid;
      my_s = s;
      my_pos = p;
      my_tok = (p >= fp && p < ctx_sh[s]) ? first + (p - fp) : -1;
    }
  } else {
    const int t0 = blk * kRows;
    if (t0 >= n_tokens) return;
    if (tid < kRows && t0 + tid < n_tokens) {
      const int tok = t0 + tid;
      const int s = find_seq(cu_new_lens, n_seqs, tok);
      const int first = cu_new_lens[s];
      my_s = s;
      my_pos = ctx_lens[s] - (cu_new_lens[s + 1] - first) + (tok - first);
      my_tok = tok;
    }
  }
  // the block-table entries go out now; the rows' data loads follow without waiting
  int bt_v = -1;
  if (tid < kRows) {
    if (my_tok >= 0 && my_pos >= 0 && my_pos < max_blocks * BS)  // else: drop
      bt_v = block_tables[(size_t)my_s * max_blocks + my_pos / BS];
    tok_sh[tid] = my_tok;
    pos_sh[tid] = my_pos;
  }
  __syncthreads();

  // ---- the rows' data: V staged in LDS, K and Q piece pairs in registers ----------------
  auto job = [&](int u, int heads, int& r, int& h, int& k) {
    k = u & 3;
    h = (u >> 2) % heads;
    r = (u >> 2) / heads;
  };
  const int n_kjobs = kRows * num_kv_heads * 4;  // (row, head, piece pair)
  const int n_qjobs = kRows * num_q_heads * 4;
  const int n_vchunks = kRows * hd / 8;          // 16-byte chunks of the 8 V rows
  u32x4_t vr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + 256 * i;
    const int r = e / (hd / 8);
    vr[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (e < n_vchunks && tok_sh[r] >= 0)
      vr[i] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(v_new + (size_t)tok_sh[r] * hd + 8 * (e - r * (hd / 8))));
  }
  u32x4_t ka = {0u, 0u, 0u, 0u}, kb = ka;
  if (tid < n_kjobs) {
    int r, g, k;
    job(tid, num_kv_heads, r, g, k);
    if (tok_sh[r] >= 0) {
      const size_t src = (size_t)tok_sh[r] * hd + g * kHeadDim + 8 * k;
      ka = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k_new + src));
      kb = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k_new + src + 32));
    }
  }
  u32x4_t qa[ROPE ? kQBatch : 1], qb[ROPE ? kQBatch : 1];
  if constexpr (ROPE) {
#pragma unroll
    for (int i = 0; i < kQBatch; ++i) {
      qa[i] = qb[i] = u32x4_t{0u, 0u, 0u, 0u};
      const int u = tid + 256 * i;
      int r, h, k;
      job(u, num_q_heads, r, h, k);
      if (q_in && u < n_qjobs && tok_sh[r] >= 0) {
        const size_t src = (size_t)tok_sh[r] * qd + h * kHeadDim + 8 * k;
        qa[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q_in + src));
        qb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q_in + src + 32));
      }
    }
  }
  if (tid < kRows) {
    int page = -1, slot = 0;
    if ((unsigned)bt_v < (unsigned)num_pages) { page = bt_v; slot = my_pos % BS; }  // bad id: drop
    page_sh[tid] = page;
    slot_sh[tid] = slot;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (tid + 256 * i < n_vchunks) *reinterpret_cast<u32x4_t*>(v_sh + 8 * (tid + 256 * i)) = vr[i];
  for (int e = tid + 512; e < n_vchunks; e += 256) {  // more than 8 KV heads
    const int r = e / (hd / 8);
    u32x4_t x = {0u, 0u, 0u, 0u};
    if (tok_sh[r] >= 0)
      x = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(v_new + (size_t)tok_sh[r] * hd + 8 * (e - r * (hd / 8))));
    *reinterpret_cast<u32x4_t*>(v_sh + 8 * e) = x;
  }
  if constexpr (ROPE) {
    // one angle per (row, pair): 8 x 32 = 256
    const int r = tid >> 5, i = tid & 31;
    const double f = inv_freq ? (double)inv_freq[i] : exp2(-(double)(2 * i) / kHeadDim * log2_theta);
    const double th = (double)pos_sh[r] * f;
    const double red = __builtin_fma(-rint(th / kTwoPi), kTwoPi, th);  // |red| <= pi
    double sn, cn;
    sincos(red, &sn, &cn);
    cos_sh[r][i] = (float)cn;
    sin_sh[r][i] = (float)sn;
  }
  __syncthreads();
  // the 8 rows fill slots 8j .. 8j+7 of one page (every thread reads the same answer)
  bool run = page_sh[0] >= 0 && slot_sh[0] % kRows == 0;
#pragma unroll
  for (int r = 1; r < kRows; ++r) run = run && page_sh[r] == page_sh[0] && slot_sh[r] == slot_sh[0] + r;

  // ---- K: thread = (row, head, piece pair k / k + 4) ---------------------------------
  auto put_k = [&](int r, int g, int k, u32x4_t a, u32x4_t b) {
    if constexpr (ROPE) rotate8(a, b, &cos_sh[r][8 * k], &sin_sh[r][8 * k]);
    uint16_t* kh = k_pool + ((size_t)page_sh[r] * num_kv_heads + g) * (kHeadDim * BS);
    *reinterpret_cast<u32x4_t*>(kh + ((size_t)k * BS + slot_sh[r]) * 8) = a;
    *reinterpret_cast<u32x4_t*>(kh + ((size_t)(k + 4) * BS + slot_sh[r]) * 8) = b;
  };
  if (tid < n_kjobs) {
    int r, g, k;
    job(tid, num_kv_heads, r, g, k);
    if (page_sh[r] >= 0) put_k(r, g, k, ka, kb);
  }
  for (int u = tid + 256; u < n_kjobs; u += 256) {  // more than 8 KV heads
    int r, g, k;
    job(u, num_kv_heads, r, g, k);
    if (page_sh[r] < 0) continue;
    const size_t src = (size_t)tok_sh[r] * hd + g * kHeadDim + 8 * k;
    put_k(r, g, k, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k_new + src)),
          __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k_new + src + 32)));
  }

  // ---- V: per (head, dim) page row ---------------------------------------------------
  if (run) {
    const size_t base = (size_t)page_sh[0] * num_kv_heads * (kHeadDim * BS) + slot_sh[0];
    for (int gd = tid; gd < hd; gd += 256) {
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < kRows; r += 2)
        w[r / 2] = (uint32_t)v_sh[r * hd + gd] | ((uint32_t)v_sh[(r + 1) * hd + gd] << 16);
      *reinterpret_cast<u32x4_t*>(v_pool + base + (size_t)gd * BS) = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  } else {
    for (int e = tid; e < kRows * hd; e += 256) {
      const int r = e / hd, gd = e - r * hd;
      const int page = page_sh[r];
      if (page < 0) continue;
      v_pool[(size_t)page * num_kv_heads * (kHeadDim * BS) + (size_t)gd * BS + slot_sh[r]] =
          v_sh[e];
    }
  }

  // ---- Q (rope only): rows of every query head, rotated even where K is dropped -------
  if constexpr (ROPE) {
    if (q_in) {
#pragma unroll
      for (int i = 0; i < kQBatch; ++i) {
        const int u = tid + 256 * i;
        int r, h, k;
        job(u, num_q_heads, r, h, k);
        if (u >= n_qjobs || tok_sh[r] < 0) continue;
        const size_t dst = (size_t)tok_sh[r] * qd + h * kHeadDim + 8 * k;
        rotate8(qa[i], qb[i], &cos_sh[r][8 * k], &sin_sh[r][8 * k]);
        *reinterpret_cast<u32x4_t*>(q_out + dst) = qa[i];
        *reinterpret_cast<u32x4_t*>(q_out + dst + 32) = qb[i];
      }
      for (int u = tid + 256 * kQBatch; u < n_qjobs; u += 256) {  // more than 32 query heads
        int r, h, k;
        job(u, num_q_heads, r, h, k);
        if (tok_sh[r] < 0) continue;
        const size_t src = (size_t)tok_sh[r] * qd + h * kHeadDim + 8 * k;
        u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q_in + src));
        u32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(q_in + src + 32));
        rotate8(a, b, &cos_sh[r][8 * k], &sin_sh[r][8 * k]);
        *reinterpret_cast<u32x4_t*>(q_out + src) = a;
        *reinterpret_cast<u32x4_t*>(q_out + src + 32) = b;
      }
    }
  }
}

template <bool ROPE>
hipError_t launch_append(const LaunchGeom& geo, const void* q_in, void* q_out, const void* k_new,
                         const void* v_new, void* k_pool, void* v_pool,
                         const int32_t* block_tables, int max_blocks,
                         const int32_t* cu_new_lens, const int32_t* ctx_lens, int n_seqs,
                         int n_new_tokens, double rope_theta, const float* inv_freq,
                         hipStream_t stream) {
  // enough blocks for either numbering (position-aligned: up to 2 (GS - 1) padding
  // blocks and one partial block per sequence), in whole groups for the XCD order
  const int gs = geo.block_size / kRows;
  const int64_t blocks = ((int64_t)n_new_tokens + kRows - 1) / kRows +
                         (n_seqs <= kFastSeqs ? (int64_t)n_seqs * 2 * gs : 0);
  const int64_t group = 8 * gs;
  const dim3 grid((unsigned)((blocks + group - 1) / group * group));
  const dim3 block(256);
  const size_t lds = (size_t)kRows * geo.num_kv_heads * kHeadDim * sizeof(uint16_t);
  auto* qi = static_cast<const uint16_t*>(q_in);
  auto* qo = static_cast<uint16_t*>(q_out);
  auto* kn = static_cast<const uint16_t*>(k_new);
  auto* vn = static_cast<const uint16_t*>(v_new);
  auto* kp = static_cast<uint16_t*>(k_pool);
  auto* vp = static_cast<uint16_t*>(v_pool);
  const double l2t = (ROPE && !inv_freq) ? log2(rope_theta) : 0.0;
  if (geo.block_size == 16) {
    hipLaunchKernelGGL((append_kernel<16, ROPE>), grid, block, lds, stream, qi, qo, kn, vn, kp,
                       vp, block_tables, max_blocks, cu_new_lens, ctx_lens, n_seqs, n_new_tokens,
                       geo.num_q_heads, geo.num_kv_heads, geo.num_pages, l2t, inv_freq);
  } else {
    hipLaunchKernelGGL((append_kernel<32, ROPE>), grid, block, lds, stream, qi, qo, kn, vn, kp,
                       vp, block_tables, max_blocks, cu_new_lens, ctx_lens, n_seqs, n_new_tokens,
                       geo.num_q_heads, geo.num_kv_heads, geo.num_pages, l2t, inv_freq);
  }
  return hipGetLastError();
}

// Copy-on-write: one workgroup per (src, dst) page pair copies the whole page of both
// pools with 16-byte loads and stores; a pair with an id outside the pool is skipped.
__global__ __launch_bounds__(256) void copy_pages_kernel(
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ src, const int32_t* __restrict__ dst, int num_pages,
    int page_chunks) {
  const int s = src[blockIdx.x], d = dst[blockIdx.x];
  if ((unsigned)s >= (unsigned)num_pages || (unsigned)d >= (unsigned)num_pages || s == d) return;
  const size_t so = (size_t)s * page_chunks, dof = (size_t)d * page_chunks;
  auto* k = reinterpret_cast<u32x4_t*>(k_pool);
  auto* v = reinterpret_cast<u32x4_t*>(v_pool);
  for (int c = threadIdx.x; c < page_chunks; c += 1024) {
    u32x4_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = c + 256 * i;
      if (ci < page_chunks) {
        a[i] = k[so + ci];
        b[i] = v[so + ci];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = c + 256 * i;
      if (ci < page_chunks) {
        k[dof + ci] = a[i];
        v[dof + ci] = b[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_copy_pages(const LaunchGeom& geo, void* k_pool, void* v_pool,
                             const int32_t* src_pages, const int32_t* dst_pages, int n,
                             hipStream_t stream) {
  const int page_chunks = geo.block_size * geo.num_kv_heads * kHeadDim / 8;  // 16-byte chunks
  hipLaunchKernelGGL(copy_pages_kernel, dim3(n), dim3(256), 0, stream,
                     static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), src_pages,
                     dst_pages, geo.num_pages, page_chunks);
  return hipGetLastError();
}

hipError_t launch_kv_append(const LaunchGeom& geo, const void* k_new, const void* v_new,
                            void* k_pool, void* v_pool, const int32_t* block_tables,
                            int max_blocks, const int32_t* cu_new_lens, const int32_t* ctx_lens,
                            int n_seqs, int n_new_tokens, hipStream_t stream) {
  return launch_append<false>(geo, nullptr, nullptr, k_new, v_new, k_pool, v_pool, block_tables,
                              max_blocks, cu_new_lens, ctx_lens, n_seqs, n_new_tokens, 0.0,
                              nullptr, stream);
}

hipError_t launch_rope_kv_append(const LaunchGeom& geo, const void* q_in, void* q_out,
                                 const void* k_new, const void* v_new, void* k_pool,
                                 void* v_pool, const int32_t* block_tables, int max_blocks,
                                 const int32_t* cu_new_lens, const int32_t* ctx_lens,
                                 int n_seqs, int n_new_tokens, double rope_theta,
                                 const float* inv_freq, hipStream_t stream) {
  return launch_append<true>(geo, q_in, q_out, k_new, v_new, k_pool, v_pool, block_tables,
                             max_blocks, cu_new_lens, ctx_lens, n_seqs, n_new_tokens, rope_theta,
                             inv_freq, stream);
}

}  // namespace pa

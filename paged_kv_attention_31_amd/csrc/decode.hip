// pa_decode: one query token per sequence attends to the sequence's paged K/V.
//
// The method ("tiny-vllm：从零构建高性能LLM推理引擎的完整指南", §PagedAttention and
// §在线Softmax; "Tiny-vLLM 实战", §算子融合): keys are read page by page through the
// block table, and softmax runs in one pass with a running maximum and a running sum
// that is rescaled whenever the maximum grows.  Decode moves every KV byte once and
// does 4 flop per byte, so the kernel is bound by HBM bandwidth (same guide,
// §推理流程: decode is memory-bound); everything below is arranged around keeping the
// HBM pipe full.
//
// Work split (stream-K).  Every (sequence s, KV head g) pair is a segment of
// tiles(ctx_s) = ceil(ctx_s / 64) tiles of 64 tokens (an empty context counts one empty
// tile).  Segments are laid end to end in (s, g) order and the whole tile stream is cut
// into contiguous ranges, one per worker wave, sized by the wave's weight (see Split), so
// the waves' shares do not depend on the length mix.  The prefix sum over the context lengths
// that this needs is computed on the device by every workgroup (the lengths never go to
// the host).  A wave streams its range tile by tile, crossing segment boundaries
// without a pause: the K/V loads of the next tile and the page ids and q of the tile
// after it are in flight while the current tile is computed.  The four query heads of
// a KV head share every K/V byte read.
//
// Per tile (wave-local, no workgroup barrier):
//   scores:  lane t owns token t.  The K page layout [Hkv][8][bs][8] makes "lane t reads
//            piece c of token t" a contiguous run over lanes, so eight 16-byte loads per
//            lane bring the lane its token's whole K row.  q (4 heads, bf16) sits in LDS
//            and is read as 16-byte broadcasts; dot products use v_dot2c_f32_bf16 (two
//            bf16 products per instruction, fp32 accumulate).
//   softmax: per head a wave max (DPP inside 16-lane rows, readlane across rows), scores
//            pre-scaled by scale*log2(e) so exponentials are exp2; the probabilities are
//            rounded to bf16 and go to LDS.
//   P.V:     the V page layout [Hkv][64][bs] gives each lane 8 consecutive tokens of one
//            dimension per 16-byte load, i.e. bf16 pairs along the token axis, so P.V is
//            again v_dot2c_f32_bf16 against the lane's 8 probabilities.  Tokens past the
//            end of the context are excluded by selection, never by multiplying by a
//            zero weight, so stale pool bytes (even NaN) cannot leak.
// A segment that lies wholly inside one wave's range is normalised and written as bf16
// by that wave.  A segment cut by range boundaries leaves one fp32 partial (running max,
// running sum, unnormalised output) per wave that touched it, and decode_merge_kernel
// combines them by log-sum-exp in ascending wave order (a fixed order: results do not
// depend on scheduling).
#include <algorithm>
#include <mutex>

#include "common.h"
#include "launch.h"

// Split-K scratch of pa_decode_noalloc: a device array of the library's own, so that call
// allocates nothing.  Each device holds its own copy until the process ends; host code
// reaches it only through the address hipGetSymbolAddress gives on that device.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_SCRATCH_BYTES];

namespace pa {

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

constexpr int kTile = 64;  // tokens per tile: one per lane for the scores

__device__ __forceinline__ int tiles_of(int ctx) { return ctx > 0 ? (ctx + kTile - 1) / kTile : 1; }

// The stream's cut into worker ranges.  Two things make equal tile counts unequal work:
// - Workgroups go to the XCDs in turn (workgroup b to XCD b mod 8), and on MI355X the
//   odd-numbered XCDs stream this kernel's loads 7-9% slower than the even ones (per-wave
//   wall-clock stamps, on several boxes and workloads).  A wave of an even workgroup
//   takes kWeightEven parts of the stream, one of an odd workgroup kWeightOdd.
// - A segment end costs a wave about half a tile (the cross-lane reductions and the
//   result's store).  The stream is measured in units: two per tile, one per segment end
//   (the unit after the segment's last tile), so a wave whose range crosses many short
//   segments gets fewer tiles.
// Range w holds the tiles whose first unit u = 2 t + seg (seg: the tile's segment index)
// lies in [U P(w) / P(E), U P(w + 1) / P(E)), with U = 2 T + S and P the prefix sum of
// the weights.  A range of three or more units holds a tile, and with at least two tiles
// per wave every range has three units.  Where segments average 32 tiles or more, their
// ends hardly matter and the weighted cut counts tiles alone (range w: [T P(w) / P(E),
// T P(w + 1) / P(E)), at least one tile each), which saves a wave the search for the end
// of its range.  With fewer than two tiles per wave, the cut is the plain equal split of
// the tiles.  The cut depends on (T, S, E) only, so the results stay deterministic.
__host__ __device__ constexpr int64_t split_prefix(int64_t w) {
  constexpr int64_t kS8 = 4 * (kWeightEven + kWeightOdd);  // one even and one odd workgroup
  const int64_t r = w % 8;
  return (w / 8) * kS8 + (r < 4 ? r * kWeightEven : 4 * kWeightEven + (r - 4) * kWeightOdd);
}
struct Split {
  int64_t T;  // tiles in the stream
  int64_t S;  // segments in the stream
  int E;      // worker waves
  __device__ bool weighted() const { return T >= 2 * (int64_t)E; }
  __device__ bool by_units() const { return weighted() && T < 32 * S; }
  __device__ int64_t units() const { return 2 * T + S; }
  // first tile of range w (equal or tile-weighted split)
  __device__ int64_t start(int w) const {
    return weighted() ? T * split_prefix(w) / split_prefix(E) : (int64_t)w * T / E;
  }
  // unit-weighted split: first unit of range w
  __device__ int64_t ustart(int w) const { return units() * split_prefix(w) / split_prefix(E); }
  // the range holding tile t of segment seg
  __device__ int holding(int64_t t, int64_t seg) const {
    if (!weighted()) return (int)(((t + 1) * E - 1) / T);
    constexpr int64_t kS8 = 4 * (kWeightEven + kWeightOdd);
    const int64_t u = by_units() ? 2 * t + seg : t;      // position in the split's measure
    const int64_t n = by_units() ? units() : T;
    const int64_t p = ((u + 1) * split_prefix(E) - 1) / n;  // its range w: P(w) <= p
    const int64_t w8 = p / kS8, rem = p - w8 * kS8;
    const int64_t w = 8 * w8 + (rem < 4 * kWeightEven ? rem / kWeightEven
                                                      : 4 + (rem - 4 * kWeightEven) / kWeightOdd);
    return (int)min(w, (int64_t)E - 1);
  }
};

__device__ __forceinline__ int readlane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// 16 bytes of K/V.  Every KV byte is read exactly once per call, so the loads are marked
// non-temporal: they stream past the caches instead of evicting lines that other data
// (block tables, q, partials) would reuse.  On MI355X this lifts the KV stream by ~8%.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}


// A position in a wave's tile stream (wave-uniform values).
struct Cursor {
  int s;          // sequence
  int g;          // KV head
  int i;          // tile within the (s, g) segment
  int ctx;        // context length of s (clamped)
  int nt;         // tiles per KV head of s
  int64_t first;  // stream index of the first tile of sequence s
  bool over;      // APPEND: ctx_lens[s] exceeds the cap (output NaN, nothing appended)
};

// K and V registers of one tile: lane t holds the K row of token t; for V, the lane holds
// 8 consecutive tokens of NV head dimensions of each of the PPT pages of the tile.
template <int BS>
struct DecodeTile {
  static constexpr int PPT = kTile / BS;  // pages per tile
  static constexpr int NV = BS / 8;       // 16-byte V loads per page (= dims per lane)
  uint4 k[8];
  uint4 v[PPT][NV];
};

// APPEND: one new token per sequence (the one at ctx_lens[s] - 1, rows k_new / v_new
// [n_seqs][Hkv][64]) is attended to in this launch: the wave that streams the segment's
// last tile takes the token's K/V from those rows (they come in through lanes 32..47 of the
// q load, so no load is added) in place of the pool slot.  The rows are written into the
// pools by decode_merge_kernel, which runs after this kernel in the same call, so no store
// joins the streaming loop and nothing in this kernel reads a slot being written.
template <int BS, bool APPEND>
__global__ __launch_bounds__(256) void decode_stream_kernel(
    uint16_t* __restrict__ out, float* __restrict__ ws_o, float2* __restrict__ ws_ml,
    int2* __restrict__ ws_desc, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
    int max_blocks, const int32_t* __restrict__ ctx_lens, int n_seqs, int ctx_cap,
    int num_pages, int num_kv_heads, int n_workers, float qk_scale,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new) {
  using Tile = DecodeTile<BS>;
  constexpr int PPT = Tile::PPT;
  constexpr int NV = Tile::NV;
  constexpr int LPR = BS / 8;    // lanes sharing one V row (one head dimension)
  constexpr int RPI = 64 / LPR;  // V rows covered by one 16-byte-per-lane load

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in an SGPR
  const int lane = tid & 63;
  const int hkv = num_kv_heads;
  const int hq = hkv * kGroup;
  // values read from LDS at a wave-uniform address, kept in SGPRs
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  // A context length as held below: clamped to [0, ctx_cap], except that with APPEND a
  // length past the cap reads ctx_cap + 1 (the sequence is then marked, not clamped:
  // its new token has no slot below the cap).
  auto ctx_code = [&](int raw) { return min(max(raw, 0), APPEND ? ctx_cap + 1 : ctx_cap); };

  __shared__ int scan_sh[257];
  // the context-length codes of the first kDecodeCtxCache sequences, read once for the
  // prefix sum and reused to locate the wave's first segment (no second global round trip)
  __shared__ int ctx_sh[kDecodeCtxCache];
  const bool ctx_cached = n_seqs <= kDecodeCtxCache;
  __shared__ int wsum_sh[kDecodeWaves];
  __shared__ uint4 q_sh[kDecodeWaves][2][kGroup][8];  // [wave][slot][head][piece]
  // probabilities of the tile as two bf16 terms, p = hi + lo: [wave][term][head][token]
  __shared__ __attribute__((aligned(16))) uint16_t p_sh[kDecodeWaves][2][kGroup][64];
  __shared__ __attribute__((aligned(16))) float fin_sh[kDecodeWaves][kGroup * kHeadDim];
  __shared__ float2 fin_ml[kDecodeWaves][kGroup];
  __shared__ uint4 kvn_sh[kDecodeWaves][2][16];  // APPEND: new K (8 pieces), then V (8 pieces)

  // ---- 1. tiles per sequence and their exclusive prefix sum over 256 chunks -----------
  const int chunk = (n_seqs + 255) / 256;
  int mine = 0;
  for (int j = 0; j < chunk; ++j) {
    const int s = tid * chunk + j;
    if (s < n_seqs) {
      const int code = ctx_code(ctx_lens[s]);
      if (ctx_cached) ctx_sh[s] = code;
      mine += tiles_of(min(code, ctx_cap));
    }
  }
  const int incl = wave_incl_scan(mine, lane);
  if (lane == 63) wsum_sh[w] = incl;
  __syncthreads();
  int before = 0;
  for (int v = 0; v < w; ++v) before += wsum_sh[v];
  scan_sh[tid] = before + incl - mine;
  if (tid == 255) scan_sh[256] = before + incl;
  __syncthreads();

  // ---- 2. this wave's range [a, b) of the tile stream ---------------------------------
  const int wid = blockIdx.x * kDecodeWaves + w;
  if (wid >= n_workers) return;  // no workgroup barrier follows
  const bool has_ws = ws_desc != nullptr;
  const int64_t n_tiles = (int64_t)uni(scan_sh[256]) * hkv;
  const int64_t n_eff = min((int64_t)n_workers, n_tiles);
  // header for the merge: stream length and the number of waves it is cut into
  if (has_ws && wid == 0 && lane == 0) ws_desc[n_workers] = make_int2((int)n_tiles, (int)n_eff);
  if (wid >= n_eff) {
    if (has_ws && lane == 0) ws_desc[wid] = make_int2(-1, 0);
    return;
  }
  const Split split{n_tiles, (int64_t)n_seqs * hkv, (int)n_eff};
  const bool units = split.by_units();
  // Position lookup: a position counts tiles (equal split) or units (weighted split).  The
  // sequences before sequence k, holding cum tiles per KV head, span hkv * cum tiles or
  // hkv * (2 cum + k) units.
  auto seq_pos = [&](int64_t cum, int64_t k) -> int64_t {
    return units ? (int64_t)hkv * (2 * cum + k) : (int64_t)hkv * cum;
  };
  struct Where {
    int s;       // sequence holding the position
    int code;    // its context-length code
    int nt;      // its tiles per KV head
    int64_t cum; // tiles per KV head before it
  };
  auto find = [&](int64_t pos) -> Where {
    // The chunk holding pos: the chunk prefix is non-decreasing, so it is the number of
    // chunk starts at or below pos, less one (lane l checks chunks 4 l .. 4 l + 3 at once).
    int n_le = 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = 4 * lane + jj;
      n_le += __popcll(__ballot(seq_pos(scan_sh[c], min(c * chunk, n_seqs)) <= pos));
    }
    const int lo = uni(n_le) - 1;
    Where wh{-1, 0, 1, uni(scan_sh[lo])};
    if (chunk == 1) {  // a chunk is one sequence: pos lies in sequence lo
      wh.s = lo;
      wh.code = uni(ctx_sh[lo]);
      wh.nt = tiles_of(min(wh.code, ctx_cap));
    }
    // else the sequence inside the chunk, 64 sequences per step
    for (int s0 = lo * chunk; wh.s < 0 && s0 < n_seqs; s0 += 64) {
      const int sj = s0 + lane;
      const int cj = sj < n_seqs ? (ctx_cached ? ctx_sh[sj] : ctx_code(ctx_lens[sj])) : 0;
      const int nj = sj < n_seqs ? tiles_of(min(cj, ctx_cap)) : 0;
      const int pre = wave_incl_scan(nj, lane);
      const uint64_t hit = __ballot(pos < seq_pos(wh.cum + pre, sj + 1));
      if (hit) {
        const int j = __ffsll((unsigned long long)hit) - 1;
        wh.s = s0 + j;
        wh.code = readlane_i(cj, j);
        wh.nt = readlane_i(nj, j);
        wh.cum += readlane_i(pre - nj, j);
        break;
      }
      wh.cum += readlane_i(pre, 63);
    }
    return wh;
  };
  // (KV head, tile) of position pos inside sequence wh; with units, a position inside a
  // tile's second unit or on a segment's end unit moves to the next tile (which may be
  // the next segment's first, i == nt)
  auto place = [&](const Where& wh, int64_t pos, int& g, int& i) {
    const int64_t off = pos - seq_pos(wh.cum, wh.s);
    if (units) {
      const int64_t segu = 2 * (int64_t)wh.nt + 1;
      g = (int)(off / segu);
      i = (int)((off - g * segu + 1) >> 1);
    } else {
      g = (int)(off / wh.nt);
      i = (int)(off - (int64_t)g * wh.nt);
    }
  };
  const int64_t pa = units ? split.ustart(wid) : split.start(wid);
  const Where wa = find(pa);
  if (wa.s < 0) return;  // unreachable: a position below the end lies in some sequence
  int ga, ia;
  place(wa, pa, ga, ia);
  const int64_t a = (int64_t)hkv * wa.cum + (int64_t)ga * wa.nt + ia;  // first tile
  int64_t b = split.start(wid + 1);                                    // one past the last
  if (units) {
    const int64_t pb = split.ustart(wid + 1);
    b = n_tiles;
    if (pb < split.units()) {
      const Where wb = find(pb);
      int gb, ib;
      place(wb, pb, gb, ib);
      b = (int64_t)hkv * wb.cum + (int64_t)gb * wb.nt + ib;
    }
  }
  const int L = (int)(b - a);
  Cursor cc{wa.s, ga, ia, min(wa.code, ctx_cap), wa.nt, (int64_t)hkv * wa.cum, wa.code > ctx_cap};
  const bool bump = ia == wa.nt;  // the first tile is the next segment's: step onto it below
  if (bump) cc.i = wa.nt - 1;
  // Context lengths of the next 64 sequences, one per lane.  A range is at most 56 * Hkv
  // tiles long (the host sizes the worker count for that) and every sequence holds at
  // least Hkv tiles, so a range touches at most 58 sequences.
  const int cache_base = cc.s;
  const int cache_ctx =
      cache_base + lane < n_seqs
          ? (ctx_cached ? ctx_sh[cache_base + lane] : ctx_code(ctx_lens[cache_base + lane]))
          : 0;
  auto advance = [&](Cursor& c) {
    if (++c.i == c.nt) {
      c.i = 0;
      if (++c.g == hkv) {
        c.g = 0;
        c.first += (int64_t)hkv * c.nt;
        ++c.s;
        const int code = readlane_i(cache_ctx, min(c.s - cache_base, 63));
        c.ctx = min(code, ctx_cap);
        c.over = code > ctx_cap;
        c.nt = tiles_of(c.ctx);
      }
    }
  };

  if (bump) advance(cc);

  const size_t head_stride = (size_t)kHeadDim * BS;  // elements of one (page, head)
  const size_t page_stride = head_stride * hkv;

  // page ids of a tile: lane l reads the entry of page (l % PPT) of the tile; pages past
  // the last block of the context repeat the last block (never read as data)
  auto load_pages = [&](const Cursor& c) -> int {
    const int last = c.ctx > 0 ? (c.ctx - 1) / BS : 0;
    const int blk = min(c.i * PPT + lane % PPT, last);
    return block_tables[(size_t)c.s * max_blocks + blk];
  };
  // q of the tile's segment: lane l (and l + 32) reads piece l % 8 of head (l % 32) / 8
  // (APPEND: lanes 32..39 read the segment's new K row, lanes 40..47 its new V row, 16 bytes
  // each; lanes 48..63 repeat the K row)
  auto load_q = [&](const Cursor& c) -> uint4 {
    if constexpr (APPEND) {
      const uint16_t* src =
          lane < 32 ? q + ((size_t)c.s * hq + c.g * kGroup) * kHeadDim + 8 * lane
                    : ((lane >> 3) == 5 ? v_new : k_new) + ((size_t)c.s * hkv + c.g) * kHeadDim +
                          8 * (lane & 7);
      return *reinterpret_cast<const uint4*>(src);
    } else {
      return reinterpret_cast<const uint4*>(q + ((size_t)c.s * hq + c.g * kGroup) * kHeadDim)
          [lane & 31];
    }
  };
  auto store_q = [&](int slot, uint4 v) {
    if (lane < 32) q_sh[w][slot][lane >> 3][lane & 7] = v;
    if constexpr (APPEND) {
      if (lane >= 32 && lane < 48) kvn_sh[w][slot][lane - 32] = v;
    }
  };
  // Issue the K/V loads of a tile.  `live` false (a tile past the end of the range)
  // points every lane at one 16-byte piece, so each load instruction fetches one line.
  // Returns true if a page id is out of range (page 0 is read instead).
  auto load_kv = [&](Tile& t, const Cursor& c, int pid, bool live) -> bool {
    int pg[PPT];
    bool bad = APPEND && c.over;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      pg[j] = readlane_i(pid, j);
      if (c.ctx == 0) pg[j] = 0;  // an empty context has no pages to name
      if ((unsigned)pg[j] >= (unsigned)num_pages) {
        bad = true;
        pg[j] = 0;
      }
    }
    int kpage = pg[0];
#pragma unroll
    for (int j = 1; j < PPT; ++j) kpage = (live && lane >= j * BS) ? pg[j] : kpage;
    const size_t hoff = (size_t)c.g * head_stride;
    const uint16_t* kb = k_pool + (size_t)kpage * page_stride + hoff + (live ? (lane % BS) * 8 : 0);
#pragma unroll
    for (int p = 0; p < 8; ++p) t.k[p] = load_stream(kb + p * BS * 8);
    const int vl = live ? (lane / LPR) * BS + (lane % LPR) * 8 : 0;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const uint16_t* vb = v_pool + (size_t)pg[j] * page_stride + hoff + vl;
#pragma unroll
      for (int i = 0; i < NV; ++i) t.v[j][i] = load_stream(vb + i * RPI * BS);
    }
    return bad;
  };

  float m[kGroup], l[kGroup], acc[NV][kGroup];
  auto reset = [&]() {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) acc[i][h] = 0.f;
    }
  };
  reset();

  // scores, online-softmax update and P.V of the tile at cursor c, held in t
  auto compute = [&](Tile& t, const Cursor& c, int slot) {
    const int nvalid = min(max(c.ctx - c.i * kTile, 0), kTile);
    if constexpr (APPEND) {
      if (c.ctx > 0 && c.i == c.nt - 1 && !c.over) {  // uniform: the tile holds the newest token
        const int pn = nvalid - 1;           // its index in the tile
        if (lane == pn) {
#pragma unroll
          for (int p = 0; p < 8; ++p) t.k[p] = kvn_sh[w][slot][p];
        }
        // V: the lanes whose 8-token run holds the token replace its element
        const int pin = pn % BS;
        const int jn = pn / BS;
        const int e = pin & 7;
        if (lane % LPR == pin / 8) {
          const uint16_t* vn = reinterpret_cast<const uint16_t*>(&kvn_sh[w][slot][8]);
#pragma unroll
          for (int j = 0; j < PPT; ++j) {
            if (j != jn) continue;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
              const uint32_t x = vn[lane / LPR + i * RPI];
              const uint32_t lo_mask = (e & 1) ? 0x0000ffffu : 0xffff0000u;
              const uint32_t ins = (e & 1) ? (x << 16) : x;
              const int wd = e >> 1;
              t.v[j][i].x = wd == 0 ? ((t.v[j][i].x & lo_mask) | ins) : t.v[j][i].x;
              t.v[j][i].y = wd == 1 ? ((t.v[j][i].y & lo_mask) | ins) : t.v[j][i].y;
              t.v[j][i].z = wd == 2 ? ((t.v[j][i].z & lo_mask) | ins) : t.v[j][i].z;
              t.v[j][i].w = wd == 3 ? ((t.v[j][i].w & lo_mask) | ins) : t.v[j][i].w;
            }
          }
        }
      }
    }
    // q comes from LDS as 16-byte broadcasts, two pieces (4 heads each) in registers at a
    // time: the reads of piece p + 2 are tied (through an empty asm) to the dot products
    // of piece p, so the compiler can neither hoist all 32 reads (128 registers) nor
    // leave a read waiting right before its use.
    int qofs = 0;
    asm volatile("" : "+s"(qofs));
    float x[kGroup] = {0.f, 0.f, 0.f, 0.f};
    uint4 qa[kGroup], qb[kGroup];
#pragma unroll
    for (int h = 0; h < kGroup; ++h) qa[h] = q_sh[w][slot][h][qofs + 0];
#pragma unroll
    for (int h = 0; h < kGroup; ++h) qb[h] = q_sh[w][slot][h][qofs + 1];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      uint4* qc = (p & 1) ? qb : qa;
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        float a = x[h];
        a = dot2(t.k[p].x, qc[h].x, a);
        a = dot2(t.k[p].y, qc[h].y, a);
        a = dot2(t.k[p].z, qc[h].z, a);
        a = dot2(t.k[p].w, qc[h].w, a);
        x[h] = a;
      }
      if (p + 2 < 8) {
        asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+s"(qofs));
#pragma unroll
        for (int h = 0; h < kGroup; ++h) qc[h] = q_sh[w][slot][h][qofs + p + 2];
      }
    }
#pragma unroll
    for (int h = 0; h < kGroup; ++h) x[h] = lane < nvalid ? x[h] * qk_scale : kNegInf;

    // Online-softmax update.  The tile maxima are wave-uniform, so the rescale of the
    // running sums and outputs is one uniform branch, skipped when no head's maximum
    // grew.  p goes to P.V as two bf16 terms, hi = bf16(p) and lo = bf16(p - hi), so
    // the weights keep 16 significant bits (one bf16 term alone, 8 bits, can move the
    // output of a row dominated by a few keys by 2^-8 of the spread of their V values);
    // the running sum adds the same hi + lo, so the output is an exact convex
    // combination of V rows.
    float mt[kGroup] = {x[0], x[1], x[2], x[3]};
    wave_max4(mt[0], mt[1], mt[2], mt[3]);
    if (mt[0] > m[0] || mt[1] > m[1] || mt[2] > m[2] || mt[3] > m[3]) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        const float mn = fmaxf(m[h], mt[h]);
        const float alpha = m[h] == mn ? 1.f : fast_exp2(m[h] - mn);  // 0 while m = -inf
        l[h] *= alpha;
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i][h] *= alpha;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      const float mref = m[h] == kNegInf ? 0.f : m[h];  // a tile with no key keeps m = -inf
      const float p = fast_exp2(x[h] - mref);           // 0 for tokens past the end
      const uint16_t ph = to_bf16(p);
      const float phf = __uint_as_float((uint32_t)ph << 16);
      const uint16_t pl = to_bf16(p - phf);
      l[h] += phf + __uint_as_float((uint32_t)pl << 16);
      p_sh[w][0][h][lane] = ph;
      p_sh[w][1][h][lane] = pl;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if (nvalid < kTile) {
      // tokens past the end may hold stale bytes (even NaN): clear them
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        const int tb = j * BS + (lane % LPR) * 8;  // tile index of this lane's first token
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          uint32_t wv[4] = {t.v[j][i].x, t.v[j][i].y, t.v[j][i].z, t.v[j][i].w};
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            if (tb + k >= nvalid) wv[k >> 1] &= (k & 1) ? 0x0000ffffu : 0xffff0000u;
          }
          t.v[j][i] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
      }
    }
    // P.V over the hi terms, then over the lo terms
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        const int tb = j * BS + (lane % LPR) * 8;
        uint4 pp[kGroup];
#pragma unroll
        for (int h = 0; h < kGroup; ++h)
          pp[h] = *reinterpret_cast<const uint4*>(&p_sh[w][part][h][tb]);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const uint4 vv = t.v[j][i];
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
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // End of a segment's part in this range: the bf16 output if the whole segment was
  // here, else an fp32 partial.  A range cuts at most two segments, its first (cut at its
  // start) and its last (cut at its end), so wave wid has two partial slots: 2 wid for
  // its first segment, 2 wid + 1 for a last segment whose first tile it holds.  The wave that holds the
  // first tile of a cut segment (its last segment) records (segment, stream index of the
  // segment's last tile) for the merge, which finds the range holding that tile
  // (Split::holding).
  // The result goes through LDS so that one 16-byte store per lane writes it (bf16: lane
  // l < 32 holds head l / 8, dims 8 (l % 8) .. +8; fp32: lane l holds head l / 16, dims
  // 4 (l % 16) .. +4), and the stores themselves are issued by the step on every tile
  // through buffer descriptors whose range is empty unless a segment ended: equal store
  // counts on every path keep the compiler's vector-memory wait counts exact, so the K/V
  // loads in flight are never waited on because of these stores.  The data they store is
  // left in acc[0][0..3] and acc[1][0..1] (reset right after).
  constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3: raw (untyped) access
  auto rsrc_none = [&]() { return __builtin_amdgcn_make_buffer_rsrc(out, 0, 0, kRsrcWord3); };
  int2 own = make_int2(-1, 0);
  auto finish = [&](const Cursor& c, bool started, bool whole, bool bad,
                    __amdgpu_buffer_rsrc_t& r_data, __amdgpu_buffer_rsrc_t& r_ml) {
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      l[h] = wave_sum(l[h]);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float a = acc[i][h];
        // the LPR lanes of a dimension are neighbours inside a quad: DPP swaps, no LDS
        a += dpp_f<kDppQuadSwap1>(a);
        if (LPR == 4) a += dpp_f<kDppQuadSwap2>(a);
        acc[i][h] = bad ? __builtin_nanf("") : a;
      }
    }
    // lanes l % LPR == 0 hold dims l / LPR + i * RPI of every head
    if (lane % LPR == 0) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h)
#pragma unroll
        for (int i = 0; i < NV; ++i) fin_sh[w][h * kHeadDim + lane / LPR + i * RPI] = acc[i][h];
    }
    // m and l are wave-uniform
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h) fin_ml[w][h] = make_float2(m[h], l[h]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int seg = c.s * hkv + c.g;
    if (whole) {
      // lane l < 32: head l / 8, dims 8 (l % 8) .. +8
      const int lw = lane & 31;
      const f32x4_t f0 = *reinterpret_cast<const f32x4_t*>(&fin_sh[w][8 * lw]);
      const f32x4_t f1 = *reinterpret_cast<const f32x4_t*>(&fin_sh[w][8 * lw + 4]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int hl = lw >> 3;
      const float lh = hl == 0 ? l[0] : hl == 1 ? l[1] : hl == 2 ? l[2] : l[3];
      const float inv = lh > 0.f ? 1.f / lh : 0.f;
      acc[0][0] = __uint_as_float(pack_bf16x2(f0[0] * inv, f0[1] * inv));
      acc[0][1] = __uint_as_float(pack_bf16x2(f0[2] * inv, f0[3] * inv));
      acc[0][2] = __uint_as_float(pack_bf16x2(f1[0] * inv, f1[1] * inv));
      acc[0][3] = __uint_as_float(pack_bf16x2(f1[2] * inv, f1[3] * inv));
      // 512 bytes: lanes 32..63 fall outside and write nothing
      r_data = __builtin_amdgcn_make_buffer_rsrc(
          out + ((size_t)c.s * hq + c.g * kGroup) * kHeadDim, 0, kGroup * kHeadDim * 2, kRsrcWord3);
    } else {
      const f32x4_t f = *reinterpret_cast<const f32x4_t*>(&fin_sh[w][4 * lane]);
      const float2 mlp = fin_ml[w][lane & 3];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // the owner records the stream index of the segment's last tile; the merge finds
      // the wave holding it
      if (started) own = make_int2(seg, (int)(c.first + (int64_t)c.g * c.nt + c.nt - 1));
      const size_t slot = 2 * (size_t)wid + (started ? 1 : 0);
      acc[0][0] = f[0];
      acc[0][1] = f[1];
      acc[0][2] = f[2];
      acc[0][3] = f[3];
      acc[1][0] = mlp.x;  // lanes 0..3: (m, l) of head lane
      acc[1][1] = mlp.y;
      r_data = __builtin_amdgcn_make_buffer_rsrc(ws_o + slot * kGroup * kHeadDim, 0,
                                                 kGroup * kHeadDim * 4, kRsrcWord3);
      // 32 bytes: lanes 4..63 fall outside and write nothing
      r_ml = __builtin_amdgcn_make_buffer_rsrc(ws_ml + slot * kGroup, 0, kGroup * 8, kRsrcWord3);
    }
  };
  // the store slot of every tile (see above): 16 bytes of output or partial per lane, and
  // (m, l) for lanes 0..3
  auto store_slot = [&](__amdgpu_buffer_rsrc_t r_data, __amdgpu_buffer_rsrc_t r_ml) {
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4_t{__float_as_uint(acc[0][0]), __float_as_uint(acc[0][1]), __float_as_uint(acc[0][2]),
                __float_as_uint(acc[0][3])},
        r_data, lane * 16, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b64(
        u32x2_t{__float_as_uint(acc[1][0]), __float_as_uint(acc[1][1])}, r_ml, lane * 8, 0, 0);
  };

  // ---- 3. stream the range ------------------------------------------------------------
  // Cursors: cc is the tile computed now, c1 the tile whose K/V loads go out now, c2 the
  // tile whose page ids and q go out now.  Past the end of the range c1 and c2 stay on
  // the last tile and their loads are the cheap `live = false` kind.
  bool seg_whole = cc.i == 0;  // this range holds the segment's first tile
  bool seg_bad = false;
  Cursor c1, c2;

  // The prologue issues its loads in the order a pipeline step does (page ids and q of
  // the tile after next, then K/V of the next tile), and the loop is unrolled by two with
  // fixed registers per parity, so the compiler's wait counts keep one tile in flight
  // behind the one being computed.
  Tile ta, tb;
  bool bad_a = false, bad_b = false;
  int pid_x, pid_y;   // page ids: x for odd tiles, y for even tiles (after the first)
  uint4 q_x, q_y;
  {
    const int pid0 = load_pages(cc);
    store_q(0, load_q(cc));
    Cursor c0 = cc;
    c1 = cc;
    if (L > 1) advance(c1);
    pid_x = load_pages(c1);
    q_x = load_q(c1);
    bad_a = load_kv(ta, c0, pid0, true);
  }
  c2 = c1;
  if (L > 2) advance(c2);

  // one pipeline step: compute tile t (buffer cur); load K/V of tile t+1 (buffer nxt,
  // page ids pid_n1, q q_n1 already loaded); load page ids and q of tile t+2
  auto step = [&](Tile& cur, bool& bad_cur, Tile& nxt, bool& bad_nxt, int& pid_n1, int& pid_n2,
                  uint4& q_n1, uint4& q_n2, int t) {
    pid_n2 = load_pages(c2);
    q_n2 = load_q(c2);
    bad_nxt = load_kv(nxt, c1, pid_n1, t + 1 < L);
    seg_bad |= bad_cur;
    compute(cur, cc, t & 1);
    const bool ends = t == L - 1 || cc.i == cc.nt - 1;
    __amdgpu_buffer_rsrc_t r_data = rsrc_none(), r_ml = rsrc_none();
    if (ends) finish(cc, seg_whole, seg_whole && cc.i == cc.nt - 1, seg_bad, r_data, r_ml);
    store_slot(r_data, r_ml);
    if (ends) {
      reset();
      seg_whole = true;
      seg_bad = false;
    }
    store_q((t + 1) & 1, q_n1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cc = c1;
    c1 = c2;
    if (t + 3 < L) advance(c2);
  };
  for (int t = 0; t < L; t += 2) {
    step(ta, bad_a, tb, bad_b, pid_x, pid_y, q_x, q_y, t);
    if (t + 1 >= L) break;
    step(tb, bad_b, ta, bad_a, pid_y, pid_x, q_y, q_x, t + 1);
  }
  if (has_ws && lane == 0) ws_desc[wid] = own;
}

// Combine the partials of every segment that range boundaries cut.  Wave wid's
// descriptor names the segment it owns (it holds the segment's first tile) and the
// stream index of the segment's last tile; with the header (stream length T, waves E)
// the wave holding that tile is w1 = Split{T, E}.holding(last), so np = w1 - wid + 1
// consecutive waves left partials for the segment: the owner in its slot 2 wid + 1, each
// later wave w in its slot 2 w.  M = max_j m_j, L = sum_j l_j 2^(m_j - M),
// out = sum_j o_j 2^(m_j - M) / L, the sums taken in ascending wave order.  Lane = head
// dimension.  The first two partials are loaded together with the descriptor (nearly every
// wave owns a cut segment, and a cut segment has at least two), so a merge needs one
// memory round trip; further partials follow four per round.
// With k_new set (pa_decode_append), each wave first writes the new K/V rows of the
// (sequence, KV head) pairs seg = wid, wid + n_workers, ... into their pool slots (position
// ctx_lens[s] - 1; nothing for an empty context, an out-of-range page id or a length past
// the cap): lanes 0..7 store the K row's 16-byte pieces, lane d the V element of dimension d.
__global__ __launch_bounds__(256) void decode_merge_kernel(
    uint16_t* __restrict__ out, const float* __restrict__ ws_o, const float2* __restrict__ ws_ml,
    const int2* __restrict__ ws_desc, int n_workers, int num_kv_heads,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ ctx_lens,
    int n_seqs, int ctx_cap, int num_pages, int block_size) {
  const int wid = blockIdx.x * kDecodeWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k_new != nullptr && wid < n_workers) {  // each (sequence, KV head) row written once
    const size_t head_stride = (size_t)kHeadDim * block_size;
    for (int seg = wid; seg < n_seqs * num_kv_heads; seg += n_workers) {
      const int s = seg / num_kv_heads;
      const int g = seg - s * num_kv_heads;
      const int raw = ctx_lens[s];
      if (raw > ctx_cap || raw <= 0) continue;  // past the cap: no slot (output is NaN)
      const int ctx = raw;
      const int page = block_tables[(size_t)s * max_blocks + (ctx - 1) / block_size];
      if ((unsigned)page >= (unsigned)num_pages) continue;
      const int slot = (ctx - 1) % block_size;
      const size_t base = ((size_t)page * num_kv_heads + g) * head_stride;
      const uint16_t* kr = k_new + (size_t)seg * kHeadDim;
      const uint16_t* vr = v_new + (size_t)seg * kHeadDim;
      if (lane < 8)
        *reinterpret_cast<uint4*>(k_pool + base + ((size_t)lane * block_size + slot) * 8) =
            *reinterpret_cast<const uint4*>(kr + 8 * lane);
      v_pool[base + (size_t)lane * block_size + slot] = vr[lane];
    }
  }
  if (wid >= n_workers || ws_desc == nullptr) return;
  // partial j of the segment wid owns: slot 2 wid + 1 for j = 0, 2 (wid + j) after
  const int n_slots = 2 * n_workers;
  auto slot_of = [&](int j) { return min(j == 0 ? 2 * wid + 1 : 2 * (wid + j), n_slots - 1); };
  // the first two partials, issued with the descriptor
  float2 mlv[4][kGroup];
  float ov[4][kGroup];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const size_t sl = (size_t)slot_of(u);
#pragma unroll
    for (int h = 0; h < kGroup; ++h) {
      mlv[u][h] = ws_ml[sl * kGroup + h];
      ov[u][h] = ws_o[(sl * kGroup + h) * kHeadDim + lane];
    }
  }
  const int2 desc = ws_desc[wid];
  const int2 hdr = ws_desc[n_workers];  // (tiles in the stream, workers)
  const int seg = desc.x;
  if (seg < 0) return;
  const int w_last = Split{hdr.x, (int64_t)n_seqs * num_kv_heads, hdr.y}.holding(desc.y, seg);
  const int np = w_last - wid + 1;
  if (np < 2) return;
  const int s = seg / num_kv_heads;
  const int g = seg - s * num_kv_heads;
  const int hq = num_kv_heads * kGroup;
  float M[kGroup], L[kGroup], O[kGroup];
#pragma unroll
  for (int h = 0; h < kGroup; ++h) {
    M[h] = fmaxf(mlv[0][h].x, mlv[1][h].x);
    L[h] = 0.f;
    O[h] = 0.f;
  }
  // maxima of the partials past the first two, 16 partials (64 (m, l) pairs) per round
  for (int b = 2; b < np; b += 16) {
    const int j = b + (lane >> 2);
    const float mj = j < np ? ws_ml[(size_t)slot_of(j) * kGroup + (lane & 3)].x : kNegInf;
    float x0 = (lane & 3) == 0 ? mj : kNegInf;
    float x1 = (lane & 3) == 1 ? mj : kNegInf;
    float x2 = (lane & 3) == 2 ? mj : kNegInf;
    float x3 = (lane & 3) == 3 ? mj : kNegInf;
    wave_max4(x0, x1, x2, x3);
    M[0] = fmaxf(M[0], x0);
    M[1] = fmaxf(M[1], x1);
    M[2] = fmaxf(M[2], x2);
    M[3] = fmaxf(M[3], x3);
  }
  // weights and sums in ascending partial order: the first two from registers, the rest
  // four per load round
  auto accumulate = [&](int count) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        if (u < count) {
          const float f = M[h] == kNegInf || mlv[u][h].x == kNegInf
                              ? 0.f
                              : fast_exp2(mlv[u][h].x - M[h]);
          L[h] += mlv[u][h].y * f;
          O[h] += f == 0.f ? ov[u][h] * 0.f : ov[u][h] * f;  // a NaN marker survives
        }
      }
    }
  };
  accumulate(2);
  for (int v = 2; v < np; v += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool live = v + u < np;
      const size_t sl = (size_t)slot_of(live ? v + u : 0);
#pragma unroll
      for (int h = 0; h < kGroup; ++h) {
        mlv[u][h] = live ? ws_ml[sl * kGroup + h] : make_float2(kNegInf, 0.f);
        ov[u][h] = live ? ws_o[(sl * kGroup + h) * kHeadDim + lane] : 0.f;
      }
    }
    accumulate(min(4, np - v));
  }
#pragma unroll
  for (int h = 0; h < kGroup; ++h)
    out[((size_t)s * hq + g * kGroup + h) * kHeadDim + lane] =
        to_bf16(L[h] > 0.f ? O[h] / L[h] : O[h]);
}

}  // namespace

DecodePlan plan_decode(int n_seqs, int max_ctx_len, int num_kv_heads, int partition_tokens,
                       int compute_units) {
  DecodePlan p{};
  const int64_t tiles_per_seq = std::max<int64_t>(1, ((int64_t)max_ctx_len + kTile - 1) / kTile);
  const int64_t n_max = (int64_t)n_seqs * num_kv_heads * tiles_per_seq;
  // the longest range W workers can get from a stream of at most n_max tiles: an even
  // workgroup's share of the weighted cut (units: two per tile, one per segment; r units
  // hold at most (r + 1) / 2 tiles), or below two tiles per wave of the equal one
  const int64_t u_max = 2 * n_max + (int64_t)n_seqs * num_kv_heads;
  auto longest = [&](int64_t w) {
    const int64_t equal = (n_max + w - 1) / w;
    if (n_max < 2 * w) return equal;
    const int64_t r = (u_max * kWeightEven + split_prefix(w) - 1) / split_prefix(w);
    const int64_t t = (n_max * kWeightEven + split_prefix(w) - 1) / split_prefix(w);
    return std::max(std::max(equal, t), (r + 1) / 2);  // whichever weighted cut applies
  };
  const int64_t max_range = (int64_t)kDecodeMaxSeqsPerRange * num_kv_heads;
  const int64_t bound = partition_tokens > 0 ? std::min<int64_t>(partition_tokens / kTile, max_range)
                                             : max_range;
  int64_t workers = partition_tokens > 0 ? (n_max + bound - 1) / bound
                                         : (int64_t)kDecodeWaves * std::max(compute_units, 1);
  // enough workers that no range exceeds the bound: start from the even share's estimate
  workers = std::max(workers, (u_max * kWeightEven + bound * (kWeightEven + kWeightOdd) - 1) /
                                  (bound * (kWeightEven + kWeightOdd)));
  workers = std::max<int64_t>(1, std::min(workers, n_max));
  while (workers < n_max && longest(workers) > bound) ++workers;
  p.n_max_tiles = n_max;
  p.workers = workers;
  p.tiles_per_worker = std::min(longest(workers), n_max);
  p.merge = workers > 1 && tiles_per_seq > 1;
  if (p.merge) {
    const int64_t slots = 2 * workers;  // two partial slots per worker
    p.ws_bytes = (size_t)slots * kGroup * (kHeadDim * sizeof(float) + sizeof(float2)) +
                 (size_t)(workers + 1) * sizeof(int2);
  }
  return p;
}

hipError_t launch_decode(const LaunchGeom& geo, const DecodePlan& plan, void* out, const void* q,
                         const void* k_pool, const void* v_pool, const int32_t* block_tables,
                         int max_blocks, const int32_t* ctx_lens, int n_seqs, int max_ctx_len,
                         float scale, void* workspace, hipStream_t stream, const void* k_new,
                         const void* v_new) {
  const float qk_scale = scale * kLog2e;
  float* ws_o = nullptr;
  float2* ws_ml = nullptr;
  int2* ws_desc = nullptr;
  if (plan.merge) {
    const size_t slots = 2 * (size_t)plan.workers;
    ws_o = static_cast<float*>(workspace);
    ws_ml = reinterpret_cast<float2*>(ws_o + slots * kGroup * kHeadDim);
    ws_desc = reinterpret_cast<int2*>(ws_ml + slots * kGroup);
  }
  const int workers = (int)plan.workers;
  const dim3 grid((unsigned)((workers + kDecodeWaves - 1) / kDecodeWaves));
  const dim3 block(256);
  const int ctx_cap = std::min<int64_t>((int64_t)max_blocks * geo.block_size, max_ctx_len);
  auto* o = static_cast<uint16_t*>(out);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kp = static_cast<const uint16_t*>(k_pool);
  auto* vp = static_cast<const uint16_t*>(v_pool);
  auto* kn = static_cast<const uint16_t*>(k_new);
  auto* vn = static_cast<const uint16_t*>(v_new);
#define PA_DECODE_LAUNCH(B, A)                                                                  \
  hipLaunchKernelGGL((decode_stream_kernel<B, A>), grid, block, 0, stream, o, ws_o, ws_ml,      \
                     ws_desc, qq, kp, vp, block_tables, max_blocks, ctx_lens, n_seqs, ctx_cap,  \
                     geo.num_pages, geo.num_kv_heads, workers, qk_scale, kn, vn)
  const bool append = k_new != nullptr;
  if (geo.block_size == 16) {
    if (append) PA_DECODE_LAUNCH(16, true); else PA_DECODE_LAUNCH(16, false);
  } else {
    if (append) PA_DECODE_LAUNCH(32, true); else PA_DECODE_LAUNCH(32, false);
  }
#undef PA_DECODE_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (!plan.merge && !append)) return e;
  // the merge of cut segments, and (appending) the new rows' pool writes
  hipLaunchKernelGGL(decode_merge_kernel, grid, block, 0, stream, o, ws_o, ws_ml, ws_desc, workers,
                     geo.num_kv_heads, kn, vn, const_cast<uint16_t*>(kp),
                     const_cast<uint16_t*>(vp), block_tables, max_blocks, ctx_lens, n_seqs,
                     ctx_cap, geo.num_pages, geo.block_size);
  return hipGetLastError();
}

}  // namespace pa

// index_score.hip -- nvfp4 index scores for gfx950.
//
// What is computed (vLLM "nvfp4_index_decode/kernel" page, compile_score_decode: page
// layout of load_tile, per-page reduction of frag_max / score_cgs, causal limit of the
// trailing query rows): for request r, query row j < QL, index head h and page
// b < ceil(L_r / 128), the maximum over the page's tokens t <= L_r - QL + j of
// q[r QL + j, h, :] . k[t, :], with k = e2m1(code) * e4m3(scale of its 16-dim group);
// -inf when the page holds no such token.
//
// Design:
//   * Every e2m1 * e4m3 product and every e4m3 query value is exact in f16, so the page
//     is dequantised exactly (one v_cvt_scalef32_pk_f16_fp4 with unit scale and one
//     packed f16 multiply per byte) and the dot products run on v_mfma_f32_16x16x32_f16
//     with exact products and fp32 accumulation.
//   * Up to 16 query columns (j, h): A = K tile (lane = token, 32 consecutive dims per
//     lane), B = the request's query rows, kept as raw e4m3 words and converted to f16 at
//     each use (v_cvt_scalef32_pk_f16_fp8, exact).  The output layout puts 4 tokens of one
//     column in a lane; masked tokens are selected to -inf (never multiplied, so garbage
//     past the sequence cannot leak), the page max is kept per lane and reduced across
//     the four lane rows once per page.  A page that every row sees whole skips the
//     causal selects.  A page (8 tiles: 128 code bytes + 1 scale word per lane,
//     non-temporal, one buffer resource) is requested whole before its first MFMA.
//   * 17-32 columns: 32 x 32 tiles (v_mfma_f32_32x32x16_f16, all columns per operand),
//     the f16 query held in registers, half the page in flight at a time; the query rows
//     reach the wave through LDS and the page maxima of a workgroup's four waves are
//     stored together (see index_score_live32).
//   * Up to 64 requests: one wave per LIVE page.  The lengths give each request's live
//     pages; all requests' live pages form one list, and wave g of the launch takes
//     entries g, g + NW, ... with NW = the waves the chip holds at once.  A wave's chain
//     is lengths (one load, shared through L2) -> table entry -> page.  Measured on
//     MI355X (32 requests, L ~ U[1024, 32768], back-to-back launches on cold pages): one
//     wave per (request, page slot) of the grid, 40 % of them past their sequence and
//     two rounds of waves: 13.9 / 19.0 us (QL 1 x H 1 / QL 8 x H 4); persistent waves
//     over contiguous shares of the list, two per SIMD: 16.2 / 19.3 us; one wave per live
//     page: 11.7 / 15.6 us.  Wave timestamps of the last: every wave starts within 1 us,
//     the pages arrive between 2.8 and 9.2 us (45 MB at ~7 TB/s), each page then takes
//     ~1.5 us of dequant and MFMA.  The query bytes are loaded before the page, tile by
//     tile, so a page's first tiles are scored while its last ones are in flight
//     (graph-timed on MI355X: 11.8 -> 11.45 us at QL 1 x H 1).  The table entries of the
//     wave's page and of its next one are read before the loop, which the compiler turns
//     into scalar loads running beside the query loads (11.3 -> 10.6 us); the next page's
//     chain after the first is then one load.
//   * More requests: one wave per (request, page slot), the table entry read after the
//     length says the page is live.
#include "uq_device.h"
#include "uq_kernels.h"


namespace uq {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kPageTokens = 128;
constexpr int kCodeBytes = 64;    // per token: 128 e2m1 codes
constexpr int kScaleBytes = 8;    // per token: one e4m3 scale per 16 dims
constexpr int kScaleRegion = kPageTokens * kCodeBytes;
constexpr int kWaves = 4;
// waves per SIMD of the scorer kernels by column tiles (at most 96 registers).  Two
// column tiles fit by keeping half a page in registers (tile T + 4 streams into the
// registers of tile T once it is dequantised) and the query as raw e4m3 words, converted
// at each use: so the QL 8 x H 4 workload's 4128 live pages get a wave each (5120 waves)
// instead of 32 of the 4096 waves at 4 per SIMD taking a second page (MI355X: 14.7 ->
// 14.1 us; with the whole page and f16 query operands 5 waves per SIMD spilled in the
// page loop, 29.7 us).
constexpr int kLiveWavesPerSimd[2] = {5, 5};

template <int sel>
__device__ __forceinline__ f16x2 fp4_pair(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, sel);
}

__device__ __forceinline__ f16x8 cat4(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// NS tile slots of a page (8: the whole page; 4: half, refilled as it is scored)
template <int NS>
struct PageT {
  i32x4 kc[NS];       // codes [16 q, 16 q + 16) of tokens 16 T + n
  uint32_t ksw[NS];   // the scale word of groups 2q, 2q + 1 of those tokens
};
using Page = PageT<8>;

// The page through one buffer resource (wave-uniform base): a lane-constant byte offset
// plus the tile's offset as the scalar offset, so the 16 loads need no per-tile address
// registers.  Non-temporal (aux bit 1).
// records = 0 gives a resource whose loads all return zero without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint8_t* pg, int records) {
  const uint64_t base = (uint64_t)pg;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0, records, 0x00020000);
}

// Tile T of a page (codes, then the scale word) at the lane offsets co / so.
template <int NS>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, uint32_t co, uint32_t so,
                                          int T, PageT<NS>& d) {
  d.kc[T % NS] = __builtin_amdgcn_raw_buffer_load_b128(rs, co, 16 * T * kCodeBytes, 2);
  d.ksw[T % NS] = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 16 * T * kScaleBytes, 2);
}

__device__ __forceinline__ uint32_t code_off(int n, int q) {
  return (uint32_t)(n * kCodeBytes + 16 * q);
}
__device__ __forceinline__ uint32_t scale_off(int n, int q) {
  return (uint32_t)(kScaleRegion + n * kScaleBytes + 4 * (q >> 1));
}

template <int NS>
__device__ __forceinline__ void load_page(const uint8_t* pg, int n, int q, PageT<NS>& d) {
  const auto rs = page_rsrc(pg, kPageTokens * (kCodeBytes + kScaleBytes));
  // tile by tile: loads return in order, so tile T can be scored as soon as its two loads
  // are back
#pragma unroll
  for (int T = 0; T < NS; ++T) {
    load_tile(rs, code_off(n, q), scale_off(n, q), T, d);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 8 e4m3 bytes (two words, low byte first) -> 8 f16 (exact)
__device__ __forceinline__ f16x8 e4m3x8_f16_pk(int w0, int w1) {
  const f16x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2 x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2 x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return cat4(x0, x1, x2, x3);
}

// Score one page: raw e4m3 query words qr (columns c = j * H + h of request r, causal
// limits lim0[ct] = last visible token of the column's row), page data d (NS tile slots;
// with NS < 8 the page's later tiles stream in through rs) at page index b.  full
// (wave-uniform): every token of the page is visible to every row, so the causal selects
// drop out of the page max.
template <int NCT, int NS>
__device__ __forceinline__ void score_page(const IndexArgs& a, PageT<NS>& d, const i32x4 (&qr)[2][2],
                                           const int (&lim0)[2], const int r, const int b,
                                           const int n, const int q, const int R, const bool full,
                                           __amdgpu_buffer_rsrc_t rs) {
  float best[2] = {-INFINITY, -INFINITY};
  const int t_page = b * kPageTokens;
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    const uint32_t sw = d.ksw[T % NS] >> (16 * (q & 1));
    const _Float16 s0h = (_Float16)e4m3_to_f<0>((int)sw), s1h = (_Float16)e4m3_to_f<1>((int)sw);
    const f16x2 s0 = f16x2{s0h, s0h}, s1 = f16x2{s1h, s1h};
    f16x8 A[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t wd = (uint32_t)d.kc[T % NS][kk];
      const f16x2 sc = kk < 2 ? s0 : s1;
      A[kk] = cat4(fp4_pair<0>(wd) * sc, fp4_pair<1>(wd) * sc, fp4_pair<2>(wd) * sc,
                   fp4_pair<3>(wd) * sc);
    }
    // a half page in registers: tile T + NS streams into the slot tile T just freed
    if constexpr (NS < 8) {
      if (T + NS < 8) load_tile(rs, code_off(n, q), scale_off(n, q), T + NS, d);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            A[kk], e4m3x8_f16_pk(qr[ct][kk >> 1][2 * (kk & 1)], qr[ct][kk >> 1][2 * (kk & 1) + 1]),
            c4, 0, 0, 0);
      if (!full) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = t_page + 16 * T + 4 * q + jj;
          best[ct] = fmaxf(best[ct], t <= lim0[ct] ? c4[jj] : -INFINITY);
        }
      } else {
        best[ct] = fmaxf(fmaxf(best[ct], fmaxf(c4[0], c4[1])), fmaxf(c4[2], c4[3]));
      }
    }
    // one tile's operands at a time (keeps the register count, and so the waves per SIMD)
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const float m = max_across_rows(best[ct]);
    int col = 16 * ct + n;
    if constexpr (NCT == 2) asm volatile("" : "+v"(col));  // the store address is built here
    if (q == 0 && col < R) {
      const int j = col / a.H, hh = col % a.H;
      a.scores[(int64_t)hh * a.s_sh + ((int64_t)r * a.QL + j) * a.s_st + b] = m;
    }
  }
}

// Query rows of request r as the B operand (columns c = j * H + h, dims 32 q + 8 kk ..),
// from the raw e4m3 bytes a lane loaded for its column (two 16-byte words per tile).
template <int NCT = 2>
__device__ __forceinline__ void load_q_raw(const IndexArgs& a, int r, int n, int q, int R,
                                           i32x4 (&raw)[2][2]) {
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    if (ct >= NCT) {
      raw[ct][0] = raw[ct][1] = i32x4{0, 0, 0, 0};
      continue;
    }
    int col = 16 * ct + n;
    // two column tiles: opaque to the optimiser, so the lane's query address is rebuilt
    // for every page rather than hoisted out of the page loop, where its two 64-bit values
    // were spilled to scratch and reloaded ahead of the query loads (one more memory
    // round trip per page; QL 8 x H 4 on MI355X: 15.9 -> 14.8 us)
    if constexpr (NCT == 2) asm volatile("" : "+v"(col));
    raw[ct][0] = raw[ct][1] = i32x4{0, 0, 0, 0};
    if (col < R) {
      const int j = col / a.H, hh = col % a.H;
      const uint8_t* src = a.q + ((int64_t)r * a.QL + j) * a.q_st + (int64_t)hh * a.q_sh + 32 * q;
      raw[ct][0] = *reinterpret_cast<const i32x4*>(src);
      raw[ct][1] = *reinterpret_cast<const i32x4*>(src + 16);
    }
  }
}

// The live-page walk for up to 64 requests.  Lane l holds request l's length and
// live-page count (b < min(ceil(L / 128), max_blocks)); the live pages of all requests, in
// request order, form a list of Tp entries, and wave gw of the NW launched takes entries
// e, e + NW, ..., calling page(live, r, b, L, pid) for each (request, page index, length,
// physical page; live = true).  So no wave exists for a page past a sequence, a wave's
// chain is length -> table entry -> page (the table entry is read only for a live page),
// and the waves of one launch all fit on the chip at once.  The waves of a workgroup hold
// consecutive entries; with kUniform every wave of it makes as many calls as its first
// wave, a wave whose entry is past the list calling with live = false (and r, b, L, pid
// meaningless), so that the page function may synchronise the workgroup.
template <bool kUniform, class PageFn>
__device__ __forceinline__ void for_live_pages(const IndexArgs& a, int64_t gw, int64_t NW,
                                               PageFn&& page) {
  const int lane = threadIdx.x & 63;
  int Ll = lane < a.num_reqs ? a.seq_lens[lane] : 0;
  Ll = Ll < 0 ? 0 : Ll;
  int pl = (Ll + kPageTokens - 1) / kPageTokens;
  pl = pl < a.max_blocks ? pl : a.max_blocks;
  int incl = pl;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d, 64);
    incl += lane >= d ? u : 0;
  }
  const int Tp = __builtin_amdgcn_readlane(incl, 63);
  // list entry e < Tp -> (request r, page b, length L)
  auto locate = [&](int e, int& r, int& b, int& L) {
    // the request holding entry e: the first lane whose inclusive count exceeds e
    r = __builtin_popcountll(__builtin_amdgcn_ballot_w64(incl <= e));
    b = e - (r > 0 ? __builtin_amdgcn_readlane(incl, r - 1) : 0);
    L = __builtin_amdgcn_readlane(Ll, r);
  };
  // the wave's first entry.  Workgroups are dealt to the 8 XCDs in turn, and the entries
  // go to them in runs of 32, so the pages of a run (one 128-byte line of
  // every score row they write) are scored under one L2.  Entries e + NW, e + 2 NW, ...
  // follow on the same XCD as long as NW is a multiple of 256.  Either way the kWaves
  // waves of a workgroup hold consecutive entries.
  const int w = (int)(gw % kWaves);
  int e = (int)gw;
  if (NW % 256 == 0) {
    const int64_t wg = gw / kWaves;
    const int x = (int)(wg % 8);
    const int i = (int)((wg / 8) * kWaves + w);  // the wave's index on its XCD
    e = 32 * (x + 8 * (i / 32)) + i % 32;
  }
  // the entry that decides the calls: the wave's own, or its workgroup's first
  int lead = kUniform ? e - w : e;
  if (lead >= Tp) return;  // wave-uniform (workgroup-uniform with kUniform)
  bool live = kUniform ? e < Tp : true;
  int r = 0, b = 0, L = 0;
  if (live) locate(e, r, b, L);
  // the table entries of this page and of the wave's next one (when the live pages
  // outnumber the waves) in one round trip, so the next page's chain after this one is
  // a single load
  int e2 = e + (int)NW;
  int r2 = 0, b2 = 0, L2 = 0;
  if (e2 < Tp) locate(e2, r2, b2, L2);
  const int id1 = live ? a.bt[(int64_t)r * a.bt_stride + b] : 0;
  const int id2 = e2 < Tp ? a.bt[(int64_t)r2 * a.bt_stride + b2] : 0;
  int pid = __builtin_amdgcn_readfirstlane(id1);
  int pid2 = __builtin_amdgcn_readfirstlane(id2);
  while (true) {
    page(live, r, b, L, pid);
    lead += (int)NW;
    if (lead >= Tp) break;  // wave-uniform (workgroup-uniform with kUniform)
    e = e2;
    live = kUniform ? e < Tp : true;
    r = r2;
    b = b2;
    L = L2;
    pid = pid2;
    e2 = e + (int)NW;
    if (e2 < Tp) {  // a third page (more than twice as many live pages as waves)
      locate(e2, r2, b2, L2);
      pid2 = __builtin_amdgcn_readfirstlane(a.bt[(int64_t)r2 * a.bt_stride + b2]);
    }
  }
}

// One wave per live page, for up to 64 requests and at most 16 query columns (H * QL):
// 16 x 16 output tiles.
template <int NCT>
__global__ __launch_bounds__(64 * kWaves, kLiveWavesPerSimd[NCT - 1]) void index_score_live(IndexArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t NW = (int64_t)gridDim.x * kWaves;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
  const int n = lane & 15, q = lane >> 4;
  const int R = a.QL * a.H;
  for_live_pages<false>(a, gw, NW, [&](bool, int r, int b, int L, int pid) {
    // the query bytes first: vector loads return in order, so with them ahead of the
    // page the first tile's MFMAs can start while the rest of the page is in flight
    i32x4 qraw[2][2];
    load_q_raw<NCT>(a, r, n, q, R, qraw);
    constexpr int NS = NCT == 2 ? 4 : 8;
    PageT<NS> cur;
    const uint8_t* pg = a.pages + (int64_t)pid * a.page_stride;
    load_page(pg, n, q, cur);
    int lim0[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int col = 16 * ct + n;
      lim0[ct] = col < R ? L - a.QL + col / a.H : -1;  // last visible token of the row
    }
    score_page<NCT, NS>(a, cur, qraw, lim0, r, b, n, q, R, (b + 1) * kPageTokens - 1 <= L - a.QL,
                        page_rsrc(pg, kPageTokens * (kCodeBytes + kScaleBytes)));
  });
}

// ---- 17-32 query columns: 32 x 32 output tiles ----
//
// One v_mfma_f32_32x32x16_f16 takes 32 tokens (A rows) against all 32 query columns (B),
// so a query operand is converted once per 32 tokens for every column, where two 16 x 16
// column tiles convert it once per 16 tokens for each half of the columns: half the
// query conversions per page (or none, with the query held in f16), the same K
// dequantisation and the same MFMA cycles.  Lane l takes token 32 T + (l % 32) of tile T
// and dims [64 h, 64 h + 64), h = l / 32: 32 code bytes and the 4 scale bytes of those
// dims; k-step s of the tile is dims 8 s .. 8 s + 8 of each half, whose scale is byte s / 2
// of the lane's scale word.  The query operand of a lane is column l % 32, the same dims.
// Output: lane l holds column l % 32 and tokens 8 (v / 4) + 4 h + v % 4 of register v.
//
// Measured on MI355X (QL 8 x H 4, 32 requests, L ~ U[1024, 32768], graph-timed on cold
// pages, one session each): two 16 x 16 column tiles 13.8 us; 32 x 32 tiles 13.5 us;
// entries dealt to XCDs in runs of 32, 13.0-13.2 us; query through LDS and grouped score
// stores, 12.3 us (query by direct buffer-to-LDS loads) and 12.1 us (by whole-line
// register loads written to LDS, as now).  Timing copies that skipped work showed where
// the rest went: no score store 11.8 us, no query load 11.8 us, half the k-steps
// 12.3-12.6 us; the query and the stores each touched 32 lines per instruction
// (coalesced in a copy: 12.4 and 12.1 us).  Not kept: the whole page in flight with two
// tiles landing in LDS (13.8 us against 13.5), or in registers with the query converted
// at each use from LDS (13.0 against 12.4): the extra conversions cost more than the
// second round trip of half a page.

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Tile T of a page: the lane's 32 code bytes (two 16-byte words) and its scale word.
struct Tile32 {
  i32x4 kc[2];
  uint32_t ksw;
};

__device__ __forceinline__ Tile32 load_tile32(__amdgpu_buffer_rsrc_t rs, uint32_t co, uint32_t so,
                                              int T) {
  Tile32 d;
  d.kc[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, co, 32 * T * kCodeBytes, 2);
  d.kc[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, co + 16, 32 * T * kCodeBytes, 2);
  d.ksw = __builtin_amdgcn_raw_buffer_load_b32(rs, so, 32 * T * kScaleBytes, 2);
  return d;
}

// The query operand of k-step s from the lane's 64 raw e4m3 bytes.
__device__ __forceinline__ f16x8 q32_operand(const i32x4 (&qr)[4], int s) {
  return e4m3x8_f16_pk(qr[s >> 1][2 * (s & 1)], qr[s >> 1][2 * (s & 1) + 1]);
}

// One tile's 32 x 32 scores: lane l gets column l % 32, rows 8 (v / 4) + 4 h + v % 4 in
// register v.
__device__ __forceinline__ f32x16 mfma_tile32(const Tile32& d, const f16x8 (&qf)[8]) {
  const int sw = (int)d.ksw;
  f32x16 c = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const _Float16 sh = (_Float16)(s < 2   ? e4m3_to_f<0>(sw)
                                   : s < 4 ? e4m3_to_f<1>(sw)
                                   : s < 6 ? e4m3_to_f<2>(sw)
                                           : e4m3_to_f<3>(sw));
    const f16x2 sc = f16x2{sh, sh};
    const uint32_t wd = (uint32_t)d.kc[s >> 2][s & 3];
    const f16x8 A = cat4(fp4_pair<0>(wd) * sc, fp4_pair<1>(wd) * sc, fp4_pair<2>(wd) * sc,
                         fp4_pair<3>(wd) * sc);
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, qf[s], c, 0, 0, 0);
  }
  return c;
}

// The tile's scores into the lane's running max.  lt: the last visible row of the tile for
// the lane's column, relative to row 4 h of the tile.
__device__ __forceinline__ void max_tile32(const f32x16& c, bool full, int lt, float& best) {
  if (!full) {
#pragma unroll
    for (int v = 0; v < 16; ++v) best = fmaxf(best, 8 * (v >> 2) + (v & 3) <= lt ? c[v] : -INFINITY);
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) best = fmaxf(best, c[v]);
  }
}

// x / d for 0 <= x < 64 and 1 <= d <= 64 with inv_d = 1 / d in float: exact, since
// (x + 1/2) / d lies at least 1 / (2 d) from every integer, far beyond the float error.
__device__ __forceinline__ int small_div(int x, float inv_d) {
  return (int)(((float)x + 0.5f) * inv_d);
}

// The query rows of request r, read whole-line: load i gives lane l the 16 bytes of row
// c = 8 i + l / 8 (columns past R read column R - 1, never used), chunk (l % 8) ^ (c % 8)
// of its 128 bytes, so each load reads 8 whole rows (8 lines, where a load of the lane's
// own 16 bytes of 32 columns touches 32 lines).  put_query32 then writes them to the
// wave's LDS block at 1024 i + 16 l: row c, slot l % 8, so the reads below are free of
// bank conflicts.
__device__ __forceinline__ void load_query32(const IndexArgs& a, int r, int R, int lane,
                                             i32x4 (&raw)[4]) {
  const uint64_t base = (uint64_t)(a.q + (int64_t)r * a.QL * a.q_st);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  // the request's query bytes (a record count past 2^32 - 1 is clamped: offsets are 32-bit)
  const int64_t span = (int64_t)(a.QL - 1) * a.q_st + (int64_t)(a.H - 1) * a.q_sh + 128;
  const int records = (int)(uint32_t)(span < 0xFFFFFFFFll ? span : 0xFFFFFFFFll);
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, records, 0x00020000);
  const int sl = lane & 7;
  int c0 = lane >> 3;
  // opaque, so the offsets are computed here for every page rather than hoisted out of
  // the page loop and spilled (a scratch reload ahead of the query loads)
  asm volatile("" : "+v"(c0));
  const float inv_h = 1.0f / (float)a.H;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 8 * i + c0 < R ? 8 * i + c0 : R - 1;
    const int j = small_div(c, inv_h), hh = c - j * a.H;
    const uint32_t off = (uint32_t)(j * a.q_st + hh * a.q_sh + 16 * (sl ^ c0));
    raw[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
  }
}

__device__ __forceinline__ void put_query32(uint8_t* blk, int lane, const i32x4 (&raw)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<i32x4*>(blk + 1024 * i + 16 * lane) = raw[i];
}

// The lane's 64 query bytes (column m, dims [64 h, 64 h + 64)) from the staged block.
__device__ __forceinline__ void read_query32(const uint8_t* blk, int m, int h, i32x4 (&qr)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    qr[i] = *reinterpret_cast<const i32x4*>(blk + 128 * m + 16 * ((4 * h + i) ^ (m & 7)));
}

// Two of the page's four tiles in registers at a time: tile T + 2 is loaded into the
// registers of tile T once T's MFMAs have read them (with the f16 query held, the whole page
// in registers needs more than the 96 registers of 5 waves per SIMD).  The page maxima
// of a workgroup's four waves (four consecutive list entries: mostly four consecutive
// pages of one request) meet in LDS and are stored together, each score row receiving 16
// contiguous bytes from four adjacent lanes where one wave per page would touch 32 lines
// with 4 bytes each.
template <int NS>
__global__ __launch_bounds__(64 * kWaves, kLiveWavesPerSimd[1]) void index_score_live32(IndexArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_q[kWaves][32 * 128];
  __shared__ float lds_best[2][kWaves][32];
  __shared__ int lds_rb[2][kWaves][2];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t NW = (int64_t)gridDim.x * kWaves;
  const int64_t gw = (int64_t)blockIdx.x * kWaves + wave;
  const int m = lane & 31, h = lane >> 5;
  const int R = a.QL * a.H;
  int par = 0;
  for_live_pages<true>(a, gw, NW, [&](bool live, int r, int b, int L, int pid) {
    float best = -INFINITY;
    if (live) {
      // the query rows first (loads return in order), then the first tiles
      uint8_t* qblk = &lds_q[wave][0];
      i32x4 qraw[4];
      load_query32(a, r, R, lane, qraw);
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* pg = a.pages + (int64_t)pid * a.page_stride;
      const auto rs = page_rsrc(pg, kPageTokens * (kCodeBytes + kScaleBytes));
      const uint32_t co = (uint32_t)(m * kCodeBytes + 32 * h);
      const uint32_t so = (uint32_t)(kScaleRegion + m * kScaleBytes + 4 * h);
      Tile32 reg[NS];
#pragma unroll
      for (int T = 0; T < NS; ++T) {
        reg[T] = load_tile32(rs, co, so, T);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the query through the wave's LDS block: its whole-line layout into the operand's
      put_query32(qblk, lane, qraw);
      i32x4 qr[4];
      read_query32(qblk, m, h, qr);
      f16x8 qf[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) qf[s] = q32_operand(qr, s);
      // last visible token of the row
      const int lim = m < R ? L - a.QL + small_div(m, 1.0f / (float)a.H) : -1;
      const bool full = (b + 1) * kPageTokens - 1 <= L - a.QL;
      const int lt0 = lim - (b * kPageTokens + 4 * h);
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const f32x16 c = mfma_tile32(reg[T % NS], qf);
        if (T + NS < 4) reg[T % NS] = load_tile32(rs, co, so, T + NS);
        max_tile32(c, full, lt0 - 32 * T, best);
        __builtin_amdgcn_sched_barrier(0);
      }
      const auto o = __builtin_amdgcn_permlane32_swap(f_bits(best), f_bits(best), false, false);
      best = fmaxf(bits_f(o[0]), bits_f(o[1]));
      int mm = m;
      asm volatile("" : "+v"(mm));  // the slot address built here, not hoisted and spilled
      if (h == 0) lds_best[par][wave][mm] = best;
    }
    if (lane == 0) {
      lds_rb[par][wave][0] = live ? r : -1;
      lds_rb[par][wave][1] = b;
    }
    // every wave of the workgroup gets here once per call (the walk is uniform); the two
    // buffers alternate, so a buffer is written again only after the barrier of the next
    // call, when every wave has read it
    __syncthreads();
    int ln = lane;
    asm volatile("" : "+v"(ln));  // the addresses below built here, not hoisted and spilled
    if (ln < 32) {
      const int k = ln & 3, col = 8 * wave + (ln >> 2);
      const int rk = lds_rb[par][k][0], bk = lds_rb[par][k][1];
      if (rk >= 0 && col < R) {
        const int j = small_div(col, 1.0f / (float)a.H), hh = col - j * a.H;
        a.scores[(int64_t)hh * a.s_sh + ((int64_t)rk * a.QL + j) * a.s_st + bk] = lds_best[par][k][col];
      }
    }
    par ^= 1;
  });
}

// One wave per (request, page slot) of the grid; waves past their sequence exit after the
// length.
template <int NCT>
__global__ __launch_bounds__(64 * kWaves, kLiveWavesPerSimd[NCT - 1]) void index_score_slots(IndexArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int per_req = (a.max_blocks + kWaves - 1) / kWaves;
  const int r = blockIdx.x / per_req;
  const int b = (blockIdx.x % per_req) * kWaves + wave;
  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[r]);
  int nblk = (L + kPageTokens - 1) / kPageTokens;
  nblk = nblk < a.max_blocks ? nblk : a.max_blocks;
  if (b >= nblk) return;  // cells of pages past the sequence are left untouched
  const int n = lane & 15, q = lane >> 4;
  const int R = a.QL * a.H;
  // the query bytes, then the table entry of a live page only (read after the length),
  // then the page
  i32x4 qraw[2][2];
  load_q_raw<NCT>(a, r, n, q, R, qraw);
  const int pid = __builtin_amdgcn_readfirstlane(a.bt[(int64_t)r * a.bt_stride + b]);
  Page cur;
  const uint8_t* pg = a.pages + (int64_t)pid * a.page_stride;
  load_page(pg, n, q, cur);
  int lim0[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int col = 16 * ct + n;
    lim0[ct] = col < R ? L - a.QL + col / a.H : -1;  // last visible token of the row
  }
  score_page<NCT, 8>(a, cur, qraw, lim0, r, b, n, q, R, (b + 1) * kPageTokens - 1 <= L - a.QL,
                     page_rsrc(pg, 0));
}

}  // namespace

hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream) {
  if (a.num_reqs <= 0) return hipSuccess;
  if (a.num_reqs <= 64 && a.cus > 0) {
    // as many waves as fit on the chip at once, never more than there can be live pages
    const int nct = a.QL * a.H > 16 ? 2 : 1;
    int64_t waves = (int64_t)kLiveWavesPerSimd[nct - 1] * 4 * a.cus;
    const int64_t most = (int64_t)a.num_reqs * a.max_blocks;
    waves = waves < most ? waves : most;
    const int64_t wgs = (waves + kWaves - 1) / kWaves;
    if (nct == 2)
      hipLaunchKernelGGL((index_score_live32<2>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, stream, a);
    else
      hipLaunchKernelGGL((index_score_live<1>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, stream, a);
    return hipGetLastError();
  }
  const int64_t per_req = (a.max_blocks + kWaves - 1) / kWaves;
  const int64_t wgs = per_req * a.num_reqs;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.QL * a.H > 16)
    hipLaunchKernelGGL((index_score_slots<2>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, stream, a);
  else
    hipLaunchKernelGGL((index_score_slots<1>), dim3((unsigned)wgs), dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uq

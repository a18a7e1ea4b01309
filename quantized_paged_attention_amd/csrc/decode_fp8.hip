// decode_fp8.hip -- paged decode over an OCP e4m3 cache (per-tensor or per-token K/V
// scales), D = 128, query groups of up to 64 rows (query rows x heads), for gfx950.
//
// What is computed (ROCm/FlyDSL PR #825 "pa_decode_tile": per-tensor fp8 K/V decode with
// a cross-workgroup partition split, per_token_kv mode, query rows and wide groups; vLLM
// "ultraquant_decode_hd256" page: strided partition -> 256-token tile-group map, softmax
// statistics of STEP F, epilogue of STEP G): for a work unit (sequence b, kv head h,
// partition p) the softmax statistics (m, l, o = v_scale * sum exp(s - m) v / l) of the
// tokens of tile-groups p, p+P, ...
//
// Design (a workgroup of W = 4 waves; KV streamed once for all of a kv head's query rows
// with head groups, once per 16 rows without):
//   * Head groups (Hk a multiple of 4, or of 2 for 33-64 rows, which take two waves per
//     kv head): the 4 waves take 4 neighbouring kv heads of one (sequence, run of
//     consecutive partitions), so they read the neighbouring head slots of the same
//     blocks together; each wave streams the run as one online softmax and
//     merges it into the statistics of the run's first partition.  Otherwise the 4 waves
//     split a group of one head's partitions and their states meet in LDS.  Either way
//     the run's other partitions are written as empty (m = -inf, l = 0), which the
//     flash-combine reduce treats as absent, and the partial rows written to HBM shrink
//     by the run length.
//   * Balanced slices (head groups with much work): one workgroup per CU, each taking an
//     equal share of all sequences' partitions, split on the device from the lengths, so
//     ragged lengths leave no tail (B=128, L ~ U[4k, 16k] on MI355X: 469 -> 409 us).
//   * Measured on MI355X: partial-row write-backs interleaved with the KV read stream
//     cost far more than their bytes (88 MB of partials: +90 us on a 480 us stream);
//     the same stores kept L2-resident cost ~4 us.  With non-temporal KV loads and whole
//     runs merged into one partial, the partials stay in L2 until the kernel ends.
//   * Query rows are carried as T row tiles (T = 1 or 2); the K/V loads, the K operand
//     and the V^T transpose are shared by the tiles, each tile has its own query
//     operand, softmax state and accumulators.  Up to 8 rows: one e4m3 hi/lo tile of 8
//     rows (below).  Head groups of 9-32 rows: f16 tiles of 16 rows (one or two), 33-64
//     rows: two waves of a workgroup stream the same kv head with 32 rows each (row
//     slices: the KV bytes come from HBM once and from the caches for the sibling wave).
//     Without head groups, e4m3 tiles up to 16 rows and one launch per 16 rows beyond.
//     B=128, Hk=8, L ~ U[4k, 16k], fused step on MI355X: 8 rows 413 us; 16 rows 435 us
//     as two e4m3 tiles, 417 us as one f16 tile; 32 rows 658 us as e4m3 row slices, 454
//     us as two f16 tiles; 64 rows 1108 / 688 us.
//   * In an e4m3 tile, QK is one 16x16x128 f8f6f4 MFMA per 16 tokens with A = the K
//     codes straight from HBM (lane = token n, head dims [32r, 32r+32)) and B = the query
//     group as an e4m3 hi/lo pair -- columns 0-7 hold hi(q s_q), 8-15 lo(q s_q), added by a DPP row
//     rotate.  s_q is a per-row power of two putting the row's largest magnitude in
//     [64, 128): the pair reproduces every bf16 element of magnitude >= 2^-2 / s_q (about
//     amax / 512 to amax / 256) exactly; smaller elements land on the e4m3 subnormal grid
//     of the lo term, an error of at most 2^-10 / s_q <= 2^-16 amax per element.
//   * K is read in whole 128-byte lines: each of a tile's two K loads covers 8 tokens x
//     the full K line (lane (r, n): token (n & 7) or 8 + (n & 7), 16-byte chunk 2r or
//     2r+1), and one DPP swap with lane n ^ 8 gives every lane chunks 2r, 2r+1 of its
//     own token n.  Measured on MI355X with a load-only kernel in this kernel's order:
//     loads of 16 tokens x half a line stream at 4.5 TB/s, of 8 tokens x whole lines at
//     6.2 TB/s.
//   * Softmax is online in exp2 units against a reference max raised (with 4 units of
//     headroom) only when a score exceeds it, p = 2^(s - ref + 8) <= 256: an e4m3 hi/lo
//     pair in columns 0-7 / 8-15 of an e4m3 tile, one f16 in an f16 tile.  Each lane
//     tests its own scores against the reference; the cross-lane row maximum is taken
//     only on a raise.  The causal mask is applied only to a tile pair that reaches past
//     the shortest row window.  With per-tensor scales the row sums of P come from one
//     more MFMA (a block of ones times P), so the sums are those of the values the PV
//     MFMA multiplies.  Measured on MI355X (B=128, Hk=8, L ~ U[4k, 16k], QG=16, fused
//     step, two e4m3 tiles): 451 -> 436 us.
//   * PV takes A = V^T: each lane pair loads 16 dims of 4 tokens with 16-byte loads, swaps
//     halves (DPP) and byte-transposes (v_perm).  In an e4m3 tile the V codes go to a
//     16x16x32 fp8 MFMA per 8 head dims untouched; in an f16 tile they are converted to
//     f16 once (exactly) and shared by the row tiles.
//   * Per-token scales (the PR's per_token_kv mode): each lane loads the K and V scale of
//     one token of its 4-token quad (a 64-byte line per tile and head) and DPP-broadcasts
//     them.  The K scale multiplies the score.  The V scale rides in P: P's pair holds
//     p * v_scale_t / v_ref, with v_ref a running wave maximum of the V scales (raised,
//     with the accumulators rescaled, only when a larger scale arrives), so the fp8
//     pair keeps its range; acc * v_ref is the true sum at the end.
//   * Loads are buffer loads through a descriptor per tile whose record count ends at
//     the sequence's last visible token (invisible tokens read as zero, no branches);
//     block ids come from a window preloaded before the stream.  The next tile pair's
//     K and V loads are issued while the current pair is computed; sched_barrier fences
//     keep that order (vector loads retire in order: a misplaced wait drains them all).
#include <type_traits>

#include "uq_device.h"
#include "uq_kernels.h"

namespace uq {
namespace {

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kTiles = 16;     // tiles of 16 tokens per tile-group
constexpr int kAuxNT = 2;      // KV loads non-temporal (buffer aux bit 1, see below)
constexpr int kAuxDevice = 16;  // device-scope coherent access (buffer aux bit 4: sc1)

struct KTile {
  i32x4 a, b;  // a: K chunk 2r + (n >> 3) of token n & 7; b: chunk 2r + 1 - (n >> 3) of token
               // 8 + (n & 7) (16-byte chunks of the 128-byte K line)
};
struct VTile {
  i32x4 a, b;  // V bytes [16 (n/2), +16) of tokens 4r + 2 (n&1) and 4r + 2 (n&1) + 1
};

// A work unit's place in the fused flash-combine of its (sequence, kv head): it streams
// `take` of the sequence's `pm` partitions that hold tokens.  When take < pm its state
// goes to slot `slot`; the sequence's units use slots lo..hi.  With balanced slices slot k
// belongs to slice k - b and is unused when that slice is empty (its share of the Tt
// partitions over N slices is nothing); Tt = 0 marks every slot of the range used.
struct FuseUnit {
  int take, pm;
  int64_t slot, lo, hi;
  int64_t Tt, N;
};

// 8 e4m3 codes (two words, low byte first) -> 8 f16 (exact)
__device__ __forceinline__ f16x8 e4m3x8_f16(uint32_t w0, uint32_t w1) {
  const h16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, false);
  const h16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w0, 1.0f, true);
  const h16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, false);
  const h16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w1, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 floats -> 8 f16 (round to nearest even)
__device__ __forceinline__ f16x8 f32x8_f16(const float (&y)[8]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  h16x2 p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_convertvector((f32x2{y[2 * i], y[2 * i + 1]}), h16x2);
  return f16x8{p[0][0], p[0][1], p[1][0], p[1][1], p[2][0], p[2][1], p[3][0], p[3][1]};
}

// Output rows of unit rows RB .. RB + 8 T - 1 (those below NR) of sequence b, kv head h
// set to zero: the flash-combine of a sequence without tokens.
template <typename QT, int T, int TR = 8>
__device__ __forceinline__ void zero_output_rows(const DecodeArgs& a, const int lane, const int b,
                                                 const int h, const int RB) {
  const int NR = a.QL * a.QG;
  constexpr int kLanesPerRow = kD * (int)sizeof(QT) / 16;
  constexpr int kRowsPerPass = 64 / kLanesPerRow;
  const int u_end = RB + TR * T < NR ? RB + TR * T : NR;
  for (int u0 = RB; u0 < u_end; u0 += kRowsPerPass) {
    const int u = u0 + lane / kLanesPerRow;
    if (u < u_end) {
      QT* dst = reinterpret_cast<QT*>(a.out) + ((int64_t)b * a.QL + u / a.QG) * a.o_ss +
                (int64_t)(h * a.QG + u % a.QG) * a.o_sh;
      *reinterpret_cast<i32x4*>(dst + (lane % kLanesPerRow) * (16 / (int)sizeof(QT))) =
          i32x4{0, 0, 0, 0};
    }
  }
}

// T: row tiles of 8 query rows (16 with F16; QL x QG <= 8 T or 16 T) from unit row RB on.
// The K/V stream, the K operand and the V^T transpose are shared by the tiles; each tile has its own query operand, softmax state,
// accumulators, QK MFMA and PV MFMAs (the pages' M-tiles for wide groups).
// One work unit of a wave: kv head h of sequence b (length L, already clamped), the
// tile-groups first_tg, first_tg + step, ... (n_tg of them) of the partitions
// [part_first, p_end) it merges.  Without FUSE it writes the merged statistics to
// partition part_first and marks the others of [part_first, p_end) empty; with FUSE it
// takes part in the flash-combine of the sequence (FuseUnit) and, as the last of the
// sequence's units, writes the output rows.
// RSPL: the wave's rows are one of a.row_splits slices of the group; the waves of a
// workgroup that share a kv head read the same KV lines, so the loads keep the default
// cache policy (the sibling waves are served from the caches), and the fused state and
// counter of the unit are the slice rsi's own.
// F16 (wide groups): row tiles of 16 rows on f16 MFMAs.  The query is one f16 term
// (exact for bf16, after a per-row power of two), K and V codes are converted to f16
// exactly once per tile and shared by the row tiles, P is f16: a 16-row tile costs the
// MFMA work of an 8-row e4m3 hi/lo tile and needs no hi/lo combine, and the K / V
// conversion is paid once for up to 32 rows.
template <typename QT, int W, bool TOK, bool HG, int T, bool FUSE = false, bool RSPL = false,
          bool F16 = false>
__device__ __forceinline__ void decode_unit(const DecodeArgs& a, const int lane, const int wave,
                                            const int b, const int h, const int L,
                                            const int part_first, const int p_end,
                                            const int first_tg, const int n_tg,
                                            const int step, const int RB, const int rsi,
                                            const FuseUnit fz = FuseUnit{}) {
  constexpr int kAux = RSPL ? 0 : kAuxNT;  // cache policy of the KV loads
  static_assert(!FUSE || HG, "the fused flash-combine is built on head groups");
  static_assert(!F16 || HG, "f16 row tiles are built on head groups");
  constexpr int kTR = F16 ? 16 : 8;  // rows per row tile
  // staging of the merged partition's bf16 output rows (8 rows of 256 bytes per tile, one
  // tile at a time; one stage per wave with head groups; fused: rows of the query dtype),
  // and the states of waves 1..W-1 handed to wave 0 (per lane and tile: 32 accumulators,
  // m_run, m_true, l)
  constexpr bool kMerge = W > 1 && !HG;
  // stage rows: 8 output rows of the query dtype (fused) or bf16, padded by 16 bytes so
  // that the 16 rows a b128 store instruction touches start in different banks
  constexpr int kStageRow = (FUSE ? (int)sizeof(QT) : 2) * kD + 16;  // bytes
  constexpr int kStageBytes = kTR * kStageRow;
  __shared__ __attribute__((aligned(16))) uint8_t o_stage[(HG ? W : 1) * kStageBytes];
  __shared__ __attribute__((aligned(16))) float st_acc[kMerge ? W - 1 : 1][T][32][64];
  __shared__ float st_ml[kMerge ? W - 1 : 1][T][3][64];
  const int r = lane >> 4, n = lane & 15;
  const int g = n & 7;
  const bool lo_col = n >= 8;
  const int crow = F16 ? n : g;  // this lane's row within a row tile

  // ---- query operands.  Byte j of lane group r holds head dim d = 32 r + j (the K
  //      operand's map after the chunk exchange).  Column g of tile t holds unit row
  //      row_base + 8 t + g = (query qj, head qh) of QL query rows x QG heads; query qj
  //      sees the tokens t < L_row (the causal window of its row)
  const int NR = a.QL * a.QG;
  // per-tensor scales (the per-token ones are applied per token below)
  const float k_scale = (!TOK && a.k_scale) ? *a.k_scale : 1.f;
  const float v_scale = (!TOK && a.v_scale) ? *a.v_scale : 1.f;
  i32x8 q_own[F16 ? 1 : T];  // hi(q s_q) in columns 0-7, lo(q s_q) in columns 8-15
  f16x8 q16[F16 ? T : 1][4];  // F16: q s_q, dims 32 r + 8 s .. + 7 for MFMA k-step s
  float qk_mul[T];
  int L_row[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int urow = RB + kTR * t + crow;
    const bool qvalid = urow < NR;
    const int qj = qvalid ? urow / a.QG : 0, qh = qvalid ? urow % a.QG : 0;
    L_row[t] = L - a.QL + 1 + qj;
    float x[32];
    const QT* qp = reinterpret_cast<const QT*>(a.q) + ((int64_t)b * a.QL + qj) * a.q_ss +
                   (int64_t)(h * a.QG + qh) * a.q_sh;
    const QT* src = qp + 32 * r;
    if constexpr (sizeof(QT) == 4) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * c + e] = v[e];
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(src + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * c + 2 * e] = bf16_to_f((uint32_t)v[e] & 0xFFFFu);
          x[8 * c + 2 * e + 1] = bf16_to_f((uint32_t)v[e] >> 16);
        }
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = max_across_rows(amax);
    if constexpr (F16) {
      // s_q = 2^(15 - E) with amax = f 2^E, f in [0.5, 1): amax * s_q in [2^14, 2^15), every
      // bf16 element above 2^-24 / s_q exact in f16
      int E = 0;
      if (amax > 0.f) {
        E = (int)((f_bits(amax) >> 23) & 0xFF) - 126;
        E = E < -100 ? -100 : E;
      }
      const float s_q = bits_f((uint32_t)(127 + 15 - E) << 23);
      qk_mul[t] = a.softmax_scale * k_scale * kLog2e / s_q;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = qvalid ? x[8 * st + e] * s_q : 0.f;
        q16[F16 ? t : 0][st] = f32x8_f16(y);
      }
      continue;
    }
    // s_q = 2^(7 - E) with amax = f 2^E, f in [0.5, 1): amax * s_q in [64, 128)
    int E = 0;
    if (amax > 0.f) {
      E = (int)((f_bits(amax) >> 23) & 0xFF) - 126;
      E = E < -100 ? -100 : E;
    }
    const float s_q = bits_f((uint32_t)(127 + 7 - E) << 23);
    qk_mul[t] = a.softmax_scale * k_scale * kLog2e / s_q;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float y0 = x[4 * w] * s_q, y1 = x[4 * w + 1] * s_q, y2 = x[4 * w + 2] * s_q,
            y3 = x[4 * w + 3] * s_q;
      int hw = cvt_pk_e4m3<false>(y0, y1, 0);
      hw = cvt_pk_e4m3<true>(y2, y3, hw);
      int lw = cvt_pk_e4m3<false>(y0 - e4m3_to_f<0>(hw), y1 - e4m3_to_f<1>(hw), 0);
      lw = cvt_pk_e4m3<true>(y2 - e4m3_to_f<2>(hw), y3 - e4m3_to_f<3>(hw), lw);
      hw = qvalid ? hw : 0;
      lw = qvalid ? lw : 0;
      q_own[F16 ? 0 : t][w] = lo_col ? lw : hw;
    }
  }

  // ---- running state across tile-groups
  // base-2 state: m_run is a reference max >= every score seen, m_true the max itself,
  // l_run the sum of 2^(s - m_run + 8)
  float m_run[T], m_true[T], l_run[T];
  f32x4 acc[T][8];
  // With per-tensor scales the sums of P come from an MFMA (lacc: every element holds the
  // column sum of the P codes over the tokens so far, in columns 0-7 the hi and in 8-15
  // the lo parts); with per-token scales P carries the V scale, so they are summed on
  // the VALU from the unscaled weights (l_run, per lane).
  constexpr bool kSumByMfma = !TOK;
  constexpr long kOnesE4m3x8 = 0x3838383838383838L;  // e4m3 1.0 in every byte
  const f16x8 kOnesF16x8 = {1, 1, 1, 1, 1, 1, 1, 1};
  f32x4 lacc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    m_run[t] = -INFINITY;
    m_true[t] = -INFINITY;
    l_run[t] = 0.f;
    lacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const uint32_t pos = (uint32_t)a.pos_stride;
  // K loads: a = token n & 7, chunk 2r + (n >> 3); b = token 8 + (n & 7), chunk
  // 2r + 1 - (n >> 3): each load reads 8 tokens x whole 128-byte K lines
  const bool hi_n = n >= 8;
  const uint32_t ka_off = (uint32_t)(n & 7) * pos + 16u * (uint32_t)(2 * r + (hi_n ? 1 : 0));
  const uint32_t kb_off = (uint32_t)(8 + (n & 7)) * pos + 16u * (uint32_t)(2 * r + (hi_n ? 0 : 1));
  // V: lane pair (2h, 2h+1) fetches dims [16h, 16h+16) of tokens 4r..4r+3 with two
  // 16-byte loads per lane (the even lane tokens 4r, 4r+1, the odd lane 4r+2, 4r+3) and
  // the pair swaps halves, so each lane ends with dims [8n, 8n+8) of all four tokens.
  const int par = n & 1;
  const uint32_t v_off = (4 * r + 2 * par) * pos + kD + 16 * (n >> 1);
  // transpose selectors: the odd lane holds its four tokens in the order 2, 3, 0, 1
  const uint32_t sel_a = par ? 0x01000504u : 0x05040100u;
  const uint32_t sel_b = par ? 0x03020706u : 0x07060302u;
  const uint8_t* head_base = a.cache + (int64_t)h * a.slot_bytes;
  const int32_t* bt_row = a.bt + (int64_t)b * a.bt_stride;
  const int bs_shift = 31 - __builtin_clz(a.block_size);

  // Block ids come in windows of 8 work tile-groups: lane i holds the id of tile i % 16
  // of tile-group w0 + i / 16 (lo) and of w0 + 4 + i / 16 (hi).  The window is loaded
  // before the stream starts, so no vector-memory wait inside the stream waits for a
  // table load (vector loads retire in order: such a wait would drain every KV load
  // issued after it).  Only a wave with more than 8 tile-groups (a partition that owns
  // several strided tile-groups) reloads it, once per 8.  Tiles past L, or past the
  // wave's tile-groups, keep id 0 and are never dereferenced.
  int win_lo, win_hi;
  auto load_window = [&](int w0) {
    auto one = [&](int k) {
      int v = 0;
      if (k < n_tg) {
        const int tok = (first_tg + k * step) * kTileGroup + 16 * (lane & 15);
        if (tok < L) v = bt_row[tok >> bs_shift];
      }
      return v;
    };
    win_lo = one(w0 + (lane >> 4));
    win_hi = one(w0 + 4 + (lane >> 4));
  };
  load_window(0);
  auto load_half_window = [&](int w0) {  // tile-groups w0 .. w0+3 into their half
    auto one = [&](int k) {
      int v = 0;
      if (k < n_tg) {
        const int tok = (first_tg + k * step) * kTileGroup + 16 * (lane & 15);
        if (tok < L) v = bt_row[tok >> bs_shift];
      }
      return v;
    };
    const int v = one(w0 + (lane >> 4));
    if (w0 & 4) win_hi = v; else win_lo = v;
  };

  // Buffer resource of tile t (0..15) of work tile-group kk (in the current window):
  // base = the tile's first slot of this head, record count = its visible tokens only
  // (0 past L or past the wave's tile-groups), so every K/V byte of an invisible token
  // reads as zero with no branch, no select and no memory access.
  auto rsrc_of = [&](int kk, int t) {
    const int idx = (kk & 3) * 16 + t;
    const int b_lo = __builtin_amdgcn_readlane(win_lo, idx);
    const int b_hi = __builtin_amdgcn_readlane(win_hi, idx);
    const int blk = (kk & 7) >= 4 ? b_hi : b_lo;
    const int tok = (first_tg + kk * step) * kTileGroup + 16 * t;
    int nvis = L - tok;
    nvis = kk >= n_tg ? 0 : (nvis < 0 ? 0 : (nvis > 16 ? 16 : nvis));
    const uint64_t base = (uint64_t)(head_base + (int64_t)blk * a.blk_stride +
                                     (int64_t)(tok & (a.block_size - 1)) * pos);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                             (short)0, __builtin_amdgcn_readfirstlane(nvis * (int)pos),
                                             0x00020000);
  };
  // Per-token scale descriptor of tile t of work tile-group kk: the tile's 16 scales of
  // this head are contiguous in the [num_blocks, Hk, block_size] tensor; the record
  // count ends at the last visible token (the others read as zero).
  auto srsrc_of = [&](int kk, int t, const float* sbase) {
    const int idx = (kk & 3) * 16 + t;
    const int b_lo = __builtin_amdgcn_readlane(win_lo, idx);
    const int b_hi = __builtin_amdgcn_readlane(win_hi, idx);
    const int blk = (kk & 7) >= 4 ? b_hi : b_lo;
    const int tok = (first_tg + kk * step) * kTileGroup + 16 * t;
    int nvis = L - tok;
    nvis = kk >= n_tg ? 0 : (nvis < 0 ? 0 : (nvis > 16 ? 16 : nvis));
    const uint64_t base = (uint64_t)(sbase + ((int64_t)blk * a.Hk + h) * a.block_size +
                                     (tok & (a.block_size - 1)));
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                             (short)0, __builtin_amdgcn_readfirstlane(nvis * 4),
                                             0x00020000);
  };
  // lane (r, n) loads the scale of token 4 r + (n & 3) of a tile
  const uint32_t s_off = 4u * (uint32_t)(4 * r + (n & 3));
  auto load_s = [&](__amdgpu_buffer_rsrc_t rs) {
    return bits_f((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, s_off, 0, kAux));
  };
  auto load_k = [&](__amdgpu_buffer_rsrc_t rs, KTile& d) {
    d.a = __builtin_amdgcn_raw_buffer_load_b128(rs, ka_off, 0, kAux);
    d.b = __builtin_amdgcn_raw_buffer_load_b128(rs, kb_off, 0, kAux);
  };
  auto load_v = [&](__amdgpu_buffer_rsrc_t rs, VTile& d) {
    d.a = __builtin_amdgcn_raw_buffer_load_b128(rs, v_off, 0, kAux);
    // the second token's offset rides in the scalar offset
    d.b = __builtin_amdgcn_raw_buffer_load_b128(rs, v_off, (int)pos, kAux);
  };

  // The stream walks tile pairs (32 tokens).  The K loads of pair i + 1 are issued as
  // soon as the QK MFMAs of pair i have read their registers and its V loads as soon as
  // the V^T transpose of pair i has read them, so one pair of KV bytes is always in
  // flight while the wave computes; the register footprint stays small enough for four
  // waves per SIMD, which is what keeps the memory system busy.  No data-dependent
  // branches except a rare wave-uniform softmax rescale.
  KTile kp[2][2];  // [pair parity][tile]: K is loaded two pairs ahead
  VTile vp[2];
  // per-token scales: K scales travel with the K loads, V scales with the V loads (issued
  // just before them, so waiting for a scale never waits for the V bytes)
  float ksc[2][2] = {{0.f, 0.f}, {0.f, 0.f}}, vsc[2] = {0.f, 0.f};
  float v_ref = 0.f, v_inv = 0.f;  // running wave maximum of |V scale| and its inverse
  {
    const auto r0 = rsrc_of(0, 0), r1 = rsrc_of(0, 1);
    load_k(r0, kp[0][0]);
    load_k(r1, kp[0][1]);
    if constexpr (TOK) {
      ksc[0][0] = load_s(srsrc_of(0, 0, a.k_scale));
      ksc[0][1] = load_s(srsrc_of(0, 1, a.k_scale));
      vsc[0] = load_s(srsrc_of(0, 0, a.v_scale));
      vsc[1] = load_s(srsrc_of(0, 1, a.v_scale));
    }
    load_v(r0, vp[0]);
    load_v(r1, vp[1]);
    const auto r2 = rsrc_of(0, 2), r3 = rsrc_of(0, 3);
    load_k(r2, kp[1][0]);
    load_k(r3, kp[1][1]);
    if constexpr (TOK) {
      ksc[1][0] = load_s(srsrc_of(0, 2, a.k_scale));
      ksc[1][1] = load_s(srsrc_of(0, 3, a.k_scale));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  for (int k = 0; k < n_tg; ++k) {
    const int tg = first_tg + k * step;
    const int tg_start = tg * kTileGroup;
#pragma unroll
    for (int pr = 0; pr < kTiles / 2; ++pr) {
      const int pair_start = tg_start + 32 * pr;
      const int pf_k = pr + 1 < kTiles / 2 ? k : k + 1;  // the next pair
      const int pf_t0 = pr + 1 < kTiles / 2 ? 2 * (pr + 1) : 0;
      const int pk_k = pr + 2 < kTiles / 2 ? k : k + 1;  // the pair after next (K)
      const int pk_t0 = pr + 2 < kTiles / 2 ? 2 * (pr + 2) : 2 * (pr + 2 - kTiles / 2);
      // rolling window: the half that will hold tile-groups k+1 .. k+4 is refilled when
      // the K prefetch first reaches tile-group k+1 (rare: only for more than 8)
      if (pr == kTiles / 2 - 2 && ((k + 1) & 3) == 0 && k + 1 >= 8 && k + 1 < n_tg)
        load_half_window(k + 1);
      // the pair boundary is a scheduling fence: the next pair's QK (and its wait for
      // K loads issued one pair earlier) must not be hoisted above this pair's PV work
      __builtin_amdgcn_sched_barrier(0);
      // ---- QK: S^T[token][column] of both tiles for every row tile, hi + lo columns
      //      added by DPP
      float s[T][2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const KTile& kt = kp[pr & 1][tt];
        // lane n < 8 keeps a (its chunk 2r) and sends b; lane n >= 8 keeps b and sends a;
        // the chunk received from lane n ^ 8 is chunk 2r + 1 of this lane's token
        i32x8 kop;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int send = hi_n ? kt.a[e] : kt.b[e];
          kop[e] = hi_n ? kt.b[e] : kt.a[e];
          kop[4 + e] = (int)f_bits(row_ror8(bits_f((uint32_t)send)));
        }
        float ksq[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (TOK) quad_values(ksc[pr & 1][tt], ksq);  // K scales of tokens 4r..4r+3
        if constexpr (F16) {
          // k-step st: dims 32 r + 8 st .. + 7 of token n (bytes 8 st .. of its chunk pair)
          f16x8 kf[4];
#pragma unroll
          for (int st = 0; st < 4; ++st)
            kf[st] = e4m3x8_f16((uint32_t)kop[2 * st], (uint32_t)kop[2 * st + 1]);
#pragma unroll
          for (int t = 0; t < T; ++t) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st)
              z = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[st], q16[F16 ? t : 0][st], z, 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) s[t][tt][j] = z[j] * (TOK ? ksq[j] * qk_mul[t] : qk_mul[t]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < T; ++t) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, q_own[F16 ? 0 : t], z, 0, 0,
                                                                  0, 127, 0, 127);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float mul = TOK ? ksq[j] * qk_mul[t] : qk_mul[t];
              s[t][tt][j] = (z[j] + row_ror8(z[j])) * mul;
            }
          }
        }
      }
      // causal window: only a pair that reaches past the shortest row window (L - QL + 1
      // tokens) has invisible tokens (wave-uniform)
      if (pair_start + 32 > L - a.QL + 1) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              s[t][tt][j] = pair_start + 16 * tt + 4 * r + j < L_row[t] ? s[t][tt][j] : -INFINITY;
      }
      // Stage order is fixed: the scheduler must not hoist the prefetch loads above the
      // instructions that free their registers, nor sink them below later waits (vector
      // loads retire in order, so a misplaced load turns a partial wait into a drain).
      __builtin_amdgcn_sched_barrier(0);
      {
        const auto rk0 = rsrc_of(pk_k, pk_t0), rk1 = rsrc_of(pk_k, pk_t0 + 1);
        load_k(rk0, kp[pr & 1][0]);
        load_k(rk1, kp[pr & 1][1]);
        if constexpr (TOK) {
          ksc[pr & 1][0] = load_s(srsrc_of(pk_k, pk_t0, a.k_scale));
          ksc[pr & 1][1] = load_s(srsrc_of(pk_k, pk_t0 + 1, a.k_scale));
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- softmax against a reference max m_run >= every score seen.  It is raised
      // (with 4 units of base-2 headroom, so raises are rare) only when a score exceeds
      // it; then the running sums are rescaled.  p * 256 = 2^(s - m_run + 8) <= 256.
      // Each lane checks its own scores; only when one exceeds the reference does the wave
      // take the row maximum across lanes (m_true, the true maximum, is kept per lane and
      // reduced across lanes once, after the stream).
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float lmx = max3f(s[t][0][0], s[t][0][1], s[t][0][2]);
        lmx = max3f(lmx, s[t][0][3], s[t][1][0]);
        lmx = max3f(lmx, s[t][1][1], s[t][1][2]);
        lmx = max3f(lmx, s[t][1][3], s[t][1][3]);
        m_true[t] = max3f(m_true[t], lmx, lmx);
        if (__builtin_amdgcn_ballot_w64(lmx > m_run[t])) {  // wave-uniform
          const float mx = max_across_rows(lmx);
          const float m_new = mx > m_run[t] ? mx + 4.f : m_run[t];
          // 0 when m_run = -inf; 1 for a row that has seen no token yet (both -inf)
          const float alpha = m_run[t] == m_new ? 1.f : fast_exp2(m_run[t] - m_new);
          if constexpr (kSumByMfma) lacc[t] *= alpha;
          else l_run[t] *= alpha;
#pragma unroll
          for (int m = 0; m < 8; ++m) acc[t][m] *= alpha;
          m_run[t] = m_new;
        }
      }
      // per-token V scales of this lane's tokens; the reference v_ref is raised (and the
      // accumulators rescaled) when a larger scale arrives, so p v_scale / v_ref <= p
      float vq[2][4];
      if constexpr (TOK) {
        quad_values(vsc[0], vq[0]);
        quad_values(vsc[1], vq[1]);
        float vmx = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) vmx = fmaxf(vmx, fabsf(vq[tt][j]));
        vmx = max_across_rows(vmx);  // equal on every lane
        if (__builtin_amdgcn_ballot_w64(vmx > v_ref)) {  // wave-uniform, rare
          const float f = v_ref / vmx;  // 0 before the first nonzero scale
#pragma unroll
          for (int t = 0; t < T; ++t)
#pragma unroll
            for (int m = 0; m < 8; ++m) acc[t][m] *= f;
          v_ref = vmx;
          v_inv = 1.f / vmx;
        }
      }
      long pop[F16 ? 1 : T];
      f16x8 p16[F16 ? T : 1];  // F16: P of tokens (tile 0: 4r..4r+3, tile 1: 16+4r..) x row n
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // a row that has seen no token (m_run = -inf) has only -inf scores: weight 0
        const float m8 = m_run[t] == -INFINITY ? 0.f : m_run[t] - 8.f;
        if constexpr (F16) {
          float y[8];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float v = fast_exp2(s[t][tt][j] - m8);
              if constexpr (!kSumByMfma) l_run[t] += v;
              if constexpr (TOK) v *= vq[tt][j] * v_inv;
              y[4 * tt + j] = v;
            }
          p16[F16 ? t : 0] = f32x8_f16(y);
          if constexpr (kSumByMfma) lacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              kOnesF16x8, p16[F16 ? t : 0], lacc[t], 0, 0, 0);
          continue;
        }
        int pw[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          float y[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            y[j] = fast_exp2(s[t][tt][j] - m8);
            if constexpr (!kSumByMfma) l_run[t] += y[j];
            if constexpr (TOK) y[j] *= vq[tt][j] * v_inv;
          }
          // the score is dead once exponentiated: its register seeds the code word
          pw[tt] = e4m3_hilo_word(y[0], y[1], y[2], y[3], lo_col, (int)f_bits(s[t][tt][0]));
        }
        pop[F16 ? 0 : t] = (long)(uint32_t)pw[0] | ((long)(uint32_t)pw[1] << 32);
        // the row sums of P as the PV MFMA sees them (hi + lo columns, combined after
        // the stream): one MFMA against a block of ones instead of 8 VALU additions
        if constexpr (kSumByMfma) lacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
            kOnesE4m3x8, pop[F16 ? 0 : t], lacc[t], 0, 0, 0);
      }

      // ---- V^T: exchange halves with the neighbouring lane, then byte-transpose 8 dims
      //      x 4 tokens per tile
      uint32_t vtr[2][8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const i32x4 va = vp[tt].a, vb = vp[tt].b;
        // keep: this lane's 8 dims of its own two tokens; send: the neighbour's 8 dims
        const uint32_t k0x = par ? va[2] : va[0], k0y = par ? va[3] : va[1];
        const uint32_t k1x = par ? vb[2] : vb[0], k1y = par ? vb[3] : vb[1];
        const uint32_t r0x = swap_adjacent(par ? va[0] : va[2]);
        const uint32_t r0y = swap_adjacent(par ? va[1] : va[3]);
        const uint32_t r1x = swap_adjacent(par ? vb[0] : vb[2]);
        const uint32_t r1y = swap_adjacent(par ? vb[1] : vb[3]);
        const uint32_t lo4[4] = {k0x, k1x, r0x, r1x}, hi4[4] = {k0y, k1y, r0y, r1y};
        transpose4x4_bytes_sel(lo4, &vtr[tt][0], sel_a, sel_b);
        transpose4x4_bytes_sel(hi4, &vtr[tt][4], sel_a, sel_b);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        if constexpr (TOK) {
          vsc[0] = load_s(srsrc_of(pf_k, pf_t0, a.v_scale));
          vsc[1] = load_s(srsrc_of(pf_k, pf_t0 + 1, a.v_scale));
        }
        const auto rv0 = rsrc_of(pf_k, pf_t0), rv1 = rsrc_of(pf_k, pf_t0 + 1);
        load_v(rv0, vp[0]);
        load_v(rv1, vp[1]);
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- PV: acc[t][m][j'] holds O^T[d = 32 r' + 8 j' + m][column n'] of row tile t
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if constexpr (F16) {
          const f16x8 vf = e4m3x8_f16(vtr[0][m], vtr[1][m]);
#pragma unroll
          for (int t = 0; t < T; ++t)
            acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, p16[F16 ? t : 0], acc[t][m], 0,
                                                              0, 0);
        } else {
          const long vop = (long)vtr[0][m] | ((long)vtr[1][m] << 32);
#pragma unroll
          for (int t = 0; t < T; ++t)
            acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(vop, pop[F16 ? 0 : t], acc[t][m],
                                                                   0, 0, 0);
        }
      }
    }

  }

  // the row maxima and sums over all lanes of the column (l_sum: equal on every lane of
  // the 8 rows' columns g and g + 8)
  float l_sum[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    m_true[t] = max_across_rows(m_true[t]);
    if constexpr (kSumByMfma) l_sum[t] = F16 ? lacc[t][0] : lacc[t][0] + row_ror8(lacc[t][0]);
    else l_sum[t] = sum_across_rows(l_run[t]);
  }

  // per-token V scales: the accumulators hold the sums in units of v_ref
  if constexpr (TOK) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[t][m] *= v_ref;
  }

  if constexpr (FUSE) {
    // ---- fused flash-combine.  A unit's state is (r, l, acc) per lane: the accumulators
    //      and the sum l hold sums of 2^(s - r) (exp2 units) with r = m_run - 8, and
    //      r = -inf (l = 0, acc = 0) for a column that saw no token.
    float ref[T], lsum[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      ref[t] = m_run[t] == -INFINITY ? -INFINITY : m_run[t] - 8.f;
      lsum[t] = l_sum[t];
    }
    if (fz.take < fz.pm) {
      // Leave the state in this unit's slot with device-scope stores (written through to
      // the point where every XCD's L2 sees them), wait for them to complete, then count
      // the unit's partitions.  The unit whose count completes the sequence merges, reading
      // the states with device-scope loads; the others are done.  (A release / acquire
      // fence pair would also write back and invalidate the whole L2 of the XCD at every
      // unit end: measured on MI355X, B=128 ctx <= 16k, that costs ~110 us per step.)
      const int RSN = a.row_splits > 1 ? a.row_splits : 1;
      auto state_rsrc = [&](int64_t k) {
        const uint64_t base = (uint64_t)(a.states + (((k * a.Hk + h) * RSN + rsi) *
                                                     a.state_tiles) * (int64_t)kStateBytes);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
        return __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, T * kStateBytes,
            0x00020000);
      };
      constexpr int kML = 8 * 64 * 16;  // byte offset of (r, l) in a tile's state
      {
        const auto rs = state_rsrc(fz.slot);
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
          for (int m = 0; m < 8; ++m)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc[t][m]), rs,
                                                   t * kStateBytes + (m * 64 + lane) * 16, 0,
                                                   kAuxDevice);
          __builtin_amdgcn_raw_buffer_store_b32(f_bits(ref[t]), rs,
                                                t * kStateBytes + kML + 4 * lane, 0, kAuxDevice);
          __builtin_amdgcn_raw_buffer_store_b32(f_bits(lsum[t]), rs,
                                                t * kStateBytes + kML + 256 + 4 * lane, 0,
                                                kAuxDevice);
        }
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the state stores have completed
      int32_t* cnt = a.counters + ((int64_t)b * a.Hk + h) * RSN + rsi;
      int old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(cnt, fz.take, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __builtin_amdgcn_readfirstlane(old);
      if (old + fz.take != fz.pm) return;  // wave-uniform: another unit finishes the sequence
      // The merge starts empty and folds in every used slot of the sequence in slot order,
      // this unit's own included (read back: its stores have completed), so the output
      // does not depend on which unit happened to finish last.
#pragma unroll
      for (int t = 0; t < T; ++t) {
        ref[t] = -INFINITY;
        lsum[t] = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // the next used slot of the range at or after k
      auto next_used = [&](int64_t k) {
        for (; k <= fz.hi; ++k) {
          if (fz.Tt > 0) {
            const int64_t sl = k - b;
            if (sl * fz.Tt / fz.N >= (sl + 1) * fz.Tt / fz.N) continue;  // empty slice
          }
          break;
        }
        return k;
      };
      auto merge = [&](int t, const f32x4* x, float rk, float lk) {
        const float M = fmaxf(ref[t], rk);
        const float fa = ref[t] == -INFINITY ? 0.f : fast_exp2(ref[t] - M);
        const float fb = rk == -INFINITY ? 0.f : fast_exp2(rk - M);
#pragma unroll
        for (int m = 0; m < 8; ++m) acc[t][m] = acc[t][m] * fa + x[m] * fb;
        lsum[t] = lsum[t] * fa + lk * fb;
        ref[t] = M;
      };
      // states two at a time (one tile) or one at a time (two tiles), all their loads
      // issued before the first use
      constexpr int U = T == 1 ? 2 : 1;
      for (int64_t k0 = next_used(fz.lo); k0 <= fz.hi;) {
        int64_t ks[U];
        ks[0] = k0;
#pragma unroll
        for (int u = 1; u < U; ++u) ks[u] = ks[u - 1] <= fz.hi ? next_used(ks[u - 1] + 1) : fz.hi + 1;
        f32x4 x[U][T][8];
        float rk[U][T], lk[U][T];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (ks[u] <= fz.hi) {
            const auto rs = state_rsrc(ks[u]);
#pragma unroll
            for (int t = 0; t < T; ++t) {
#pragma unroll
              for (int m = 0; m < 8; ++m)
                x[u][t][m] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rs, t * kStateBytes + (m * 64 + lane) * 16, 0, kAuxDevice));
              rk[u][t] = bits_f(__builtin_amdgcn_raw_buffer_load_b32(
                  rs, t * kStateBytes + kML + 4 * lane, 0, kAuxDevice));
              lk[u][t] = bits_f(__builtin_amdgcn_raw_buffer_load_b32(
                  rs, t * kStateBytes + kML + 256 + 4 * lane, 0, kAuxDevice));
            }
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (ks[u] <= fz.hi)
#pragma unroll
            for (int t = 0; t < T; ++t) merge(t, x[u][t], rk[u][t], lk[u][t]);
        k0 = ks[U - 1] <= fz.hi ? next_used(ks[U - 1] + 1) : fz.hi + 1;
      }
      if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // ---- output rows: o = v_scale acc / l (0 without tokens), hi and lo columns added;
    //      the rows go through this wave's LDS stage so that each is written whole
    uint8_t* stage = o_stage + wave * kStageBytes;
    constexpr int kRowBytes = kD * (int)sizeof(QT);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int nrow = NR - RB - kTR * t < kTR ? NR - RB - kTR * t : kTR;
      if (nrow <= 0) break;  // wave-uniform
      const float inv = v_scale / (lsum[t] > 0.f ? lsum[t] : 1.f);
      if (t > 0) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // the previous tile's stage reads are done
        __builtin_amdgcn_wave_barrier();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float o[8];
#pragma unroll
        for (int m = 0; m < 8; ++m)
          o[m] = (F16 ? acc[t][m][j] : acc[t][m][j] + row_ror8(acc[t][m][j])) * inv;
        uint8_t* row = stage + n * kStageRow;
        if (n < nrow) {
          if constexpr (sizeof(QT) == 4) {
            *reinterpret_cast<f32x4*>(row + 4 * (32 * r + 8 * j)) = f32x4{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<f32x4*>(row + 4 * (32 * r + 8 * j + 4)) = f32x4{o[4], o[5], o[6], o[7]};
          } else {
            *reinterpret_cast<i32x4*>(row + 2 * (32 * r + 8 * j)) =
                i32x4{(int)pack_bf16x2(o[0], o[1]), (int)pack_bf16x2(o[2], o[3]),
                      (int)pack_bf16x2(o[4], o[5]), (int)pack_bf16x2(o[6], o[7])};
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      constexpr int kLanesPerRow = kRowBytes / 16;
      constexpr int kRowsPerPass = 64 / kLanesPerRow;
#pragma unroll
      for (int c = 0; c < kTR / kRowsPerPass; ++c) {
        const int i = c * kRowsPerPass + lane / kLanesPerRow;  // stage row
        if (i < nrow) {
          const int urow = RB + kTR * t + i;
          QT* dst = reinterpret_cast<QT*>(a.out) + ((int64_t)b * a.QL + urow / a.QG) * a.o_ss +
                    (int64_t)(h * a.QG + urow % a.QG) * a.o_sh;
          const int chunk = lane % kLanesPerRow;
          *reinterpret_cast<i32x4*>(reinterpret_cast<uint8_t*>(dst) + 16 * chunk) =
              *reinterpret_cast<const i32x4*>(stage + i * kStageRow + 16 * chunk);
        }
      }
    }
    return;
  }
  // ---- merge the W wave states into partition part_first: a lane's state belongs to
  //      its column (query head), so the merge is lane-local once the states meet in LDS
  float l_tot[T];
#pragma unroll
  for (int t = 0; t < T; ++t) l_tot[t] = l_sum[t];
  if constexpr (kMerge) {
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) st_acc[wave - 1][t][4 * m + j][lane] = acc[t][m][j];
        st_ml[wave - 1][t][0][lane] = m_run[t];
        st_ml[wave - 1][t][1][lane] = m_true[t];
        st_ml[wave - 1][t][2][lane] = l_tot[t];
      }
    }
    __syncthreads();
    if (wave > 0) return;
  }
  const int64_t row0 = (((int64_t)b * a.Hk + h) * a.P + part_first) * NR;
  uint8_t* stage = o_stage + (HG ? wave : 0) * kStageBytes;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    // statistics relative to the true maximum M over the workgroup's tokens
    float M = m_true[t];
    if constexpr (kMerge) {
#pragma unroll
      for (int w = 1; w < W; ++w) M = fmaxf(M, st_ml[w - 1][t][1][lane]);
    }
    // 0 for a wave without tokens of this row (m_run = -inf), and for every wave when the
    // row saw no token in the workgroup (M = -inf: an empty state m = -inf, l = 0)
    const float f0 = M == -INFINITY ? 0.f : fast_exp2(m_run[t] - 8.f - M);
    float l_all = l_tot[t] * f0;
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[t][m] *= f0;
    if constexpr (kMerge) {
#pragma unroll
      for (int w = 1; w < W; ++w) {
        const float fw = M == -INFINITY ? 0.f : fast_exp2(st_ml[w - 1][t][0][lane] - 8.f - M);
        l_all += st_ml[w - 1][t][2][lane] * fw;
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[t][m][j] += st_acc[w - 1][t][4 * m + j][lane] * fw;
      }
    }
    const float inv = v_scale / (l_all > 0.f ? l_all : 1.f);
    // rows RB + kTR t .. RB + kTR t + nrow - 1 of this partition's partial
    const int nrow = NR - RB - kTR * t < kTR ? NR - RB - kTR * t : kTR;
    if (nrow <= 0) break;  // wave-uniform
    // Every lane joins the DPP exchange (lanes of the lo columns feed the hi columns).
    // The bf16 rows go through LDS so that the partial is written with whole-line
    // stores: written from registers directly it would be 16-byte pieces at 64-byte
    // stride, and such scattered partial-line writes slow the concurrent KV stream.
    if (t > 0) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // the previous tile's stage reads are done
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      i32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float o0 =
            (F16 ? acc[t][2 * e][j] : acc[t][2 * e][j] + row_ror8(acc[t][2 * e][j])) * inv;
        const float o1 =
            (F16 ? acc[t][2 * e + 1][j] : acc[t][2 * e + 1][j] + row_ror8(acc[t][2 * e + 1][j])) *
            inv;
        w[e] = (int)pack_bf16x2(o0, o1);
      }
      if (n < nrow) *reinterpret_cast<i32x4*>(stage + n * kStageRow + 2 * (32 * r + 8 * j)) = w;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done
    __builtin_amdgcn_wave_barrier();
    const int nbytes = nrow * kD * 2;  // contiguous partial rows of this tile
    uint16_t* out = a.part_o + (row0 + RB + kTR * t) * kD;
#pragma unroll
    for (int c = 0; c < kTR / 4; ++c) {
      const int byte = c * 1024 + 16 * lane;  // of the nrow contiguous 256-byte rows
      if (byte < nbytes)
        *reinterpret_cast<i32x4*>(reinterpret_cast<uint8_t*>(out) + byte) =
            *reinterpret_cast<const i32x4*>(stage + (byte >> 8) * kStageRow + (byte & 255));
    }
    if (n < nrow && r == 0) {
      a.part_m[row0 + RB + kTR * t + n] = M * kLn2;
      a.part_l[row0 + RB + kTR * t + n] = l_all;
    }
  }
  // the workgroup's other partitions that hold tokens: empty states
  for (int pe = part_first + 1 + r; pe < p_end; pe += 4) {
    const int64_t prow = (((int64_t)b * a.Hk + h) * a.P + pe) * NR;
    const int u_end = RB + kTR * T < NR ? RB + kTR * T : NR;
    for (int u = RB + n; u < u_end; u += 16) {
      a.part_m[prow + u] = -INFINITY;
      a.part_l[prow + u] = 0.f;
    }
  }
}



// The decode kernel: which units a workgroup's waves stream.
//   BAL (balanced slices, head groups only): workgroup = (group of W kv heads, slice s of
//     N); the slice is an equal share of all sequences' partitions, streamed as one unit
//     per sequence it touches.  One workgroup per CU, so the kernel is compiled for one
//     wave per SIMD (AGPRs available, no spills).
//   HG: workgroup = (group of W kv heads, sequence, run); wave w streams kv head W g + w
//     over the run's partitions, so the W waves read neighbouring slots of the same
//     blocks together.
//   Otherwise: workgroup = (kv head, sequence, group of W runs) with the W runs split over
//     the waves and merged in LDS.
template <typename QT, int W, bool TOK, bool HG, int T, bool BAL, bool FUSE, bool RSPL,
          bool F16>
__global__ __launch_bounds__(64 * W, T == 1 && !F16 ? (BAL ? 1 : 3) : (BAL && F16 && T == 1 ? 1 : 2)) void decode_fp8_kernel(
    DecodeArgs a) {
  static_assert(!BAL || HG, "balanced slices are built on head groups");
  static_assert(!FUSE || HG, "the fused flash-combine is built on head groups");
  static_assert(!RSPL || HG, "row slices are built on head groups");
  static_assert(!F16 || HG, "f16 row tiles are built on head groups");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t item = blockIdx.x;
  // Row slices (RSPL): the W waves take W / RS kv heads x RS slices of the rows (16 each,
  // or 32 with f16 row tiles; wave w: head w / RS, slice w % RS); otherwise W heads (head
  // groups) or one.
  const int RS = RSPL ? a.row_splits : 1;
  const int HPW = HG ? W / RS : 1;  // kv heads per workgroup
  const int rsi = RSPL ? wave % RS : 0;
  const int RB = a.row_base + (F16 ? 32 : 16) * rsi;
  const int hw = RSPL ? wave / RS : wave;  // this wave's head within the workgroup
  // a slice past the group's rows: nothing to compute or write; head-group waves never
  // synchronise, so the wave may leave at once
  if (RSPL && RB >= a.QL * a.QG) return;
  const int nhs = HG ? a.Hk / HPW : a.Hk;
  if constexpr (BAL) {
    {
      // Balanced slices: the partitions of all sequences, in sequence order, form one list
      // of Tt entries; slice s of N takes entries [s Tt / N, (s + 1) Tt / N), so every
      // workgroup streams the same number of partitions however ragged the lengths are.
      // A slice that crosses a sequence boundary is streamed as one unit per sequence.
      const int hh = (int)(item % nhs) * HPW + hw;
      const int64_t slice = item / nhs, N = a.balanced_items;
      auto parts_of = [&](int bb) {  // partitions of sequence bb that hold tokens
        int Lb = a.seq_lens[bb];
        Lb = Lb < 0 ? 0 : (Lb > a.max_seq_len ? a.max_seq_len : Lb);
        const int ntb = (Lb + kTileGroup - 1) / kTileGroup;
        return a.P < ntb ? a.P : ntb;
      };
      // Lane l holds sequences [l per, (l + 1) per) (per <= 16: the launcher takes this
      // path for B <= 1024 only); all their lengths are loaded at once, so finding the
      // slice costs one memory round trip.
      const int per = (a.B + 63) >> 6;
      int pm[16];
      int lsum = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int q = lane * per + i;
        pm[i] = i < per && q < a.B ? parts_of(q) : 0;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) lsum += pm[i];
      int incl = lsum;  // inclusive prefix sum over the lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(incl, d, 64);
        incl += lane >= d ? u : 0;
      }
      const int64_t Tt = __builtin_amdgcn_readlane(incl, 63);
      const int64_t s0 = slice * Tt / N, s1 = (slice + 1) * Tt / N;
      // fused: the sequences without tokens b = slice, slice + N, ... get zero output rows
      // from this slice (after its stream, or at once when the slice is empty)
      auto zero_empty = [&]() {
        if constexpr (FUSE) {
          for (int64_t bz = slice; bz < a.B; bz += N)
            if (parts_of((int)bz) == 0)
              zero_output_rows<QT, T, F16 ? 16 : 8>(a, lane, (int)bz, hh, RB);
        }
      };
      if (s0 >= s1) {  // workgroup-uniform
        zero_empty();
        return;
      }
      // the lane, then the sequence within it, holding entry s0, and s0's partition index
      const int ln = __builtin_popcountll(__builtin_amdgcn_ballot_w64((int64_t)incl <= s0));
      int64_t off = s0 - (__builtin_amdgcn_readlane(incl, ln) - __builtin_amdgcn_readlane(lsum, ln));
      int bb = ln * per;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = __builtin_amdgcn_readlane(pm[i], ln);
        if (i < per && off >= v && bb + 1 < a.B) {
          off -= v;
          ++bb;
        } else {
          break;
        }
      }
      int64_t left = s1 - s0;
      int p_lo = (int)off;
      int64_t e = s0;  // list entry of (bb, p_lo)
      for (; left > 0 && bb < a.B; ++bb, p_lo = 0) {
        int Lb = __builtin_amdgcn_readfirstlane(a.seq_lens[bb]);
        Lb = Lb < 0 ? 0 : (Lb > a.max_seq_len ? a.max_seq_len : Lb);
        const int ntb = (Lb + kTileGroup - 1) / kTileGroup;
        const int pm = a.P < ntb ? a.P : ntb;
        const int take = (int)(left < pm - p_lo ? left : pm - p_lo);
        if (take <= 0) continue;
        FuseUnit fz{};
        if constexpr (FUSE) {
          // the slices holding the sequence's first and last entries: owner(x) =
          // ceil((x + 1) N / Tt) - 1; unit (bb, slice) keeps its state in slot slice + bb
          // (one-to-one: a later slice never holds an earlier sequence)
          const int64_t first = e - p_lo, last = first + pm - 1;
          fz.take = take;
          fz.pm = pm;
          fz.slot = slice + bb;
          fz.lo = ((first + 1) * N + Tt - 1) / Tt - 1 + bb;
          fz.hi = ((last + 1) * N + Tt - 1) / Tt - 1 + bb;
          fz.Tt = Tt;
          fz.N = N;
        }
        decode_unit<QT, W, TOK, HG, T, FUSE, RSPL, F16>(a, lane, wave, bb, hh, Lb, p_lo,
                                                        p_lo + take, p_lo, take, 1, RB, rsi, fz);
        left -= take;
        e += take;
      }
      zero_empty();
      return;
    }
  }
  const int h = (int)(item % nhs) * HPW + (HG ? hw : 0);
  const int b = (int)((item / nhs) % a.B);
  const int grp = (int)(item / ((int64_t)nhs * a.B));

  int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);  // wave-uniform
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int ntg = (L + kTileGroup - 1) / kTileGroup;
  // Partitions that hold tokens: p < pmax.  The workgroup owns partitions
  // [part_first, p_end): with one tile-group per partition a run of consecutive ones per
  // wave (up to R = run_len), else one partition (with its strided tile-groups) per wave.
  // The W wave states are merged into the statistics of partition part_first and the
  // workgroup's other partitions are written as empty (m = -inf, l = 0).  The
  // flash-combine of the reduce gives the same result as for separate partitions, and
  // the partial rows written to HBM shrink up to W * R times.
  const int pmax = a.P < ntg ? a.P : ntg;
  const int R = a.run_len > 0 ? a.run_len : 1;
  if constexpr (FUSE) {
    // a sequence without tokens: zero output rows from the first workgroup of its heads
    if (pmax == 0) {
      if (grp == 0) zero_output_rows<QT, T, F16 ? 16 : 8>(a, lane, b, h, RB);
      return;
    }
  }
  int part_first, p_end, first_tg, n_tg, step;
  if (HG && a.run_len > 0) {
    // this sequence's pmax partitions in G nearly equal runs of at most R; every wave
    // streams the whole run for its own kv head
    const int G = (pmax + R - 1) / R;
    if (grp >= G) return;  // workgroup-uniform: nothing written, never read
    part_first = (int)((int64_t)grp * pmax / G);
    p_end = (int)((int64_t)(grp + 1) * pmax / G);
    first_tg = part_first;
    n_tg = p_end - part_first;
    step = 1;
  } else if (HG) {
    // partition grp (its strided tile-groups) for each wave's kv head
    part_first = grp;
    if (part_first >= pmax) return;  // workgroup-uniform
    p_end = part_first + 1;
    first_tg = part_first;
    n_tg = (ntg - first_tg + a.P - 1) / a.P;
    n_tg = n_tg < a.TGPP ? n_tg : a.TGPP;
    step = a.P;
  } else if (a.run_len > 0) {
    // this sequence's pmax partitions in G nearly equal groups of at most W * R, and a
    // group's m partitions nearly equally over its W waves (no wave idles at the merge
    // for a whole run)
    const int G = (pmax + W * R - 1) / (W * R);
    if (grp >= G) return;  // workgroup-uniform: nothing written, never read
    part_first = (int)((int64_t)grp * pmax / G);
    p_end = (int)((int64_t)(grp + 1) * pmax / G);
    const int m = p_end - part_first;
    first_tg = part_first + wave * m / W;
    n_tg = part_first + (wave + 1) * m / W - first_tg;
    step = 1;
  } else {
    part_first = grp * W;
    if (part_first >= pmax) return;  // workgroup-uniform: nothing written, never read
    p_end = part_first + W < pmax ? part_first + W : pmax;
    // partition part_first + wave owns the strided tile-groups p, p + P, ...
    first_tg = part_first + wave;
    n_tg = first_tg < pmax ? (ntg - first_tg + a.P - 1) / a.P : 0;
    n_tg = n_tg < a.TGPP ? n_tg : a.TGPP;
    step = a.P;
  }

  FuseUnit fz{};
  if constexpr (FUSE) {
    // units (b, grp) keep their states in slots b * runs + grp, grp < the sequence's count
    // of workgroups (runs of partitions, or single partitions with strided tile-groups)
    const int G = a.run_len > 0 ? (pmax + R - 1) / R : pmax;
    fz.take = p_end - part_first;
    fz.pm = pmax;
    fz.slot = (int64_t)b * a.runs + grp;
    fz.lo = (int64_t)b * a.runs;
    fz.hi = fz.lo + G - 1;
    fz.Tt = 0;
    fz.N = 1;
  }
  decode_unit<QT, W, TOK, HG, T, FUSE, RSPL, F16>(a, lane, wave, b, h, L, part_first, p_end,
                                                  first_tg, n_tg, step, RB, rsi, fz);
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, bool q_is_f32, bool tok_scales,
                             hipStream_t stream) {
  constexpr int W = 4;
  const bool hg = a.head_groups != 0;
  // Row tiles: up to 8 rows, one e4m3 hi/lo tile of 8 rows; head groups with 9-32 rows
  // take one or two f16 tiles of 16 rows, and split 33-64 rows over 2 waves of a
  // workgroup (row slices, one launch).  Without head groups, e4m3 tiles up to 16 rows,
  // and a wider group runs in passes of 16 rows, each reading the KV stream once.
  const int rows = a.QL * a.QG;
  if (rows > 64) return hipErrorInvalidValue;
  const bool f16 = hg && rows > 8;
  const int RS = a.row_splits > 1 ? a.row_splits : 1;
  if (RS != (f16 && rows > 32 ? 2 : 1)) return hipErrorInvalidValue;
  const int HPW = hg ? W / RS : 1;  // kv heads per workgroup
  if (hg && a.Hk % HPW != 0) return hipErrorInvalidValue;
  // balanced slices hold up to 16 sequence lengths per lane
  if (a.balanced_items > 0 && (!hg || a.B > 1024)) return hipErrorInvalidValue;
  // tiles per wave: e4m3 up to 8 rows in one tile, 16 in two; f16 up to 16 rows in one
  const int T = f16 ? (rows <= 16 ? 1 : 2) : (rows <= 8 ? 1 : 2);
  const bool fuse = a.fused != 0;
  if (fuse && (!hg || !a.out || !a.counters || !a.states || a.state_tiles != T))
    return hipErrorInvalidValue;
  const int R = a.run_len > 0 ? a.run_len : 1;
  // BAL: one workgroup per (HPW kv heads, slice); HG: per (HPW kv heads, sequence, run);
  // else per (kv head, sequence, W runs)
  const int64_t groups = hg ? (int64_t)a.runs
                            : ((int64_t)a.runs * R + (int64_t)W * R - 1) / ((int64_t)W * R);
  const int64_t items = a.balanced_items > 0 ? (int64_t)a.balanced_items * (a.Hk / HPW)
                                             : groups * a.B * (hg ? a.Hk / HPW : a.Hk);
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)items), block(64 * W);
  const bool bal = hg && a.balanced_items > 0;
  auto go = [&](auto kernel, const DecodeArgs& p) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, p);
  };
  // one instantiation per (query type, per-token scales, order, row tiles, fused, slices)
  auto pick = [&](auto qt, auto tok, const DecodeArgs& p) {
    using QT = decltype(qt);
    constexpr bool TOK = decltype(tok)::value;
    if (f16 && T == 1) {  // one f16 row tile (9-16 rows), head groups
      if (bal) {
        if (fuse) go(decode_fp8_kernel<QT, W, TOK, true, 1, true, true, false, true>, p);
        else go(decode_fp8_kernel<QT, W, TOK, true, 1, true, false, false, true>, p);
      } else {
        if (fuse) go(decode_fp8_kernel<QT, W, TOK, true, 1, false, true, false, true>, p);
        else go(decode_fp8_kernel<QT, W, TOK, true, 1, false, false, false, true>, p);
      }
    } else if (f16) {  // f16 row tiles (two per wave), head groups
      if (RS > 1) {
        if (bal) {
          if (fuse) go(decode_fp8_kernel<QT, W, TOK, true, 2, true, true, true, true>, p);
          else go(decode_fp8_kernel<QT, W, TOK, true, 2, true, false, true, true>, p);
        } else {
          if (fuse) go(decode_fp8_kernel<QT, W, TOK, true, 2, false, true, true, true>, p);
          else go(decode_fp8_kernel<QT, W, TOK, true, 2, false, false, true, true>, p);
        }
      } else {
        if (bal) {
          if (fuse) go(decode_fp8_kernel<QT, W, TOK, true, 2, true, true, false, true>, p);
          else go(decode_fp8_kernel<QT, W, TOK, true, 2, true, false, false, true>, p);
        } else {
          if (fuse) go(decode_fp8_kernel<QT, W, TOK, true, 2, false, true, false, true>, p);
          else go(decode_fp8_kernel<QT, W, TOK, true, 2, false, false, false, true>, p);
        }
      }
    } else if (bal) {
      if (fuse) {
        if (T == 1) go(decode_fp8_kernel<QT, W, TOK, true, 1, true, true, false, false>, p);
        else go(decode_fp8_kernel<QT, W, TOK, true, 2, true, true, false, false>, p);
      } else {
        if (T == 1) go(decode_fp8_kernel<QT, W, TOK, true, 1, true, false, false, false>, p);
        else go(decode_fp8_kernel<QT, W, TOK, true, 2, true, false, false, false>, p);
      }
    } else if (hg) {
      if (fuse) {
        if (T == 1) go(decode_fp8_kernel<QT, W, TOK, true, 1, false, true, false, false>, p);
        else go(decode_fp8_kernel<QT, W, TOK, true, 2, false, true, false, false>, p);
      } else {
        if (T == 1) go(decode_fp8_kernel<QT, W, TOK, true, 1, false, false, false, false>, p);
        else go(decode_fp8_kernel<QT, W, TOK, true, 2, false, false, false, false>, p);
      }
    } else {
      if (T == 1) go(decode_fp8_kernel<QT, W, TOK, false, 1, false, false, false, false>, p);
      else go(decode_fp8_kernel<QT, W, TOK, false, 2, false, false, false, false>, p);
    }
  };
  const int pass_rows = f16 ? 32 * RS : 16;
  for (int rb = 0; rb < rows; rb += pass_rows) {
    DecodeArgs p = a;
    p.row_base = rb;
    p.row_splits = RS;
    if (tok_scales) {
      if (q_is_f32) pick(float{}, std::true_type{}, p); else pick(uint16_t{}, std::true_type{}, p);
    } else {
      if (q_is_f32) pick(float{}, std::false_type{}, p); else pick(uint16_t{}, std::false_type{}, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace uq

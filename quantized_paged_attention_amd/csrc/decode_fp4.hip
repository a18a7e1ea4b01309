// decode_fp4.hip -- paged decode over an fp4 e2m1 cache with e4m3 scales per 32 head
// dims, D = 256, query groups of up to 16 heads, with the query rotated in-kernel into
// the cache's randomized-Hadamard key domain.  gfx950.
//
// What is computed (vLLM "ultraquant_decode_hd256" page: AoS slot of K codes, K scales,
// V codes, V scales; strided partition -> 256-token tile-group map; fused Walsh-Hadamard
// query rotation of STEP B'; online softmax of STEP F; partition epilogue of STEP G):
// for a unit (sequence b, kv head h, partition p) the softmax statistics of the tokens of
// tile-groups p, p+P, ...:  m = max s, l = sum exp(s - m), o = sum exp(s - m) v / l, with
// s = softmax_scale * (q R) . k, R = diag(signs) H / 16 (H the natural-order Sylvester
// Hadamard matrix), k and v decoded as e2m1(code) * e4m3(scale of its 32-dim group).
//
// Design (one workgroup of four waves per unit):
//   * Every product e2m1 * e4m3 is exact in f16 (at most 6 significant bits, magnitudes
//     in [2^-10, 2688]), so K and V are dequantised exactly with one v_cvt_scalef32_pk_
//     f16_fp4 (its scale operand applies only a power of two, so it is left at 1) and one
//     packed f16 multiply per byte, and QK / PV run on v_mfma_f32_16x16x32_f16.
//   * The rotated query is computed once per workgroup: wave w transforms heads 4w..4w+3
//     (lane = 16 consecutive dims of a head: four butterfly stages in registers, four
//     across lanes), scales each row by a power of two that puts its largest magnitude in
//     [2^14, 2^15) (full f16 precision, no overflow), and leaves it in LDS in f16.
//   * Wave w streams tokens [64w, 64w + 64) of each of the unit's tile-groups, 32 tokens
//     per step.  QK: A = K (lane = token, 64 consecutive head dims per lane, dims permuted
//     identically in the query operand), B = query (lane = head).  Softmax is online in
//     exp2 units with a reference that is only moved when a score exceeds it (ballot).
//     PV: A = P straight from the QK output layout, B = V with lane = 16 consecutive head
//     dims of 8 tokens; a nibble transpose (v_bfi) pairs the two tokens of each f16x2 so
//     that every B register is one convert and one multiply by the tokens' scale pair.
//   * The four waves' (m, l, acc) are merged in LDS; the normalised rows are written as
//     bf16 with whole-row stores.
#include "uq_device.h"
#include "uq_kernels.h"

namespace uq {
namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 256;
constexpr int kW = 4;          // waves per workgroup, 64 tokens of a tile-group each
constexpr int kKScales = 128;  // slot offsets: K codes 0, K scales 128, V codes 136,
constexpr int kVCodes = 136;   // V scales 264 (one e4m3 byte per 32 head dims)
constexpr int kVScales = 264;

template <int sel>
__device__ __forceinline__ f16x2 fp4_pair(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, sel);
}

__device__ __forceinline__ f16x2 splat_h(float s) {
  const _Float16 h = (_Float16)s;
  return f16x2{h, h};
}

__device__ __forceinline__ f16x8 cat4(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// e4m3 byte `byte_idx` (0..3, runtime) of a word -> float
__device__ __forceinline__ float e4m3_byte(uint32_t word, int byte_idx) {
  return e4m3_to_f<0>((int)(word >> (8 * byte_idx)));
}

struct Chunk {
  i32x4 kc[2][2];      // K codes of tiles 0, 1 (e4m3 scales: bytes [32q, +16), [32q + 16,
                       // +16); UE8M0 scales: bytes [16q, +16) and [64 + 16q, +16))
  uint32_t ksw[2][2];  // K scale words of tiles 0, 1 (UE8M0: all 8 scale bytes)
  i32x2 vc[8];      // V codes, dims 16 n .. 16 n + 15, of the 8 tokens of the PV k-slots
  uint32_t vsw[8];  // V scale word of those tokens
};

// Byte offsets of a lane's loads inside a 16-token tile (constant for the kernel).
struct LaneOffsets {
  uint32_t k;      // K codes of token n, bytes 32 q ..
  uint32_t ks;     // K scale word of token n holding groups 2q, 2q + 1
  uint32_t v[4];   // V codes of token 4q + e, dims 16 n ..
  uint32_t vs[4];  // V scale word of token 4q + e holding group n / 2
};

// Buffer resource of the 16-token tile starting at token `tok` (a multiple of 16) of kv
// head h: base = the tile's first slot of the head, record count = its visible tokens
// only, so every byte of a token past L reads as zero with no branch and no access.
// The block id comes from lane (tok / bs - blk_lo) of the wave's preloaded ids.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const DecodeArgs& a, int ids,
                                                           int blk_lo, int tok, int L, int h,
                                                           int bs_shift) {
  const int blk = tok >> bs_shift;
  const int phys = __builtin_amdgcn_readlane(ids, blk - blk_lo);
  int nvis = L - tok;
  nvis = nvis < 0 ? 0 : (nvis > 16 ? 16 : nvis);
  const uint64_t base = (uint64_t)(a.cache + (int64_t)phys * a.blk_stride +
                                   (int64_t)(tok & (a.block_size - 1)) * a.pos_stride +
                                   (int64_t)h * a.slot_bytes);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0,
                                           __builtin_amdgcn_readfirstlane(nvis * a.pos_stride),
                                           0x00020000);
}

template <bool UE>
__device__ __forceinline__ Chunk load_chunk(const DecodeArgs& a, int n, int q, int ids,
                                            int blk_lo, int t0, int L, int h, int bs_shift) {
  Chunk c;
  LaneOffsets o;  // (recomputed per step: cheaper than keeping 10 registers live)
  {
    const uint32_t pos = (uint32_t)a.pos_stride;
    // e4m3 scales: 64 consecutive dims per lane, dequantised before the MFMA; UE8M0: one
    // 32-dim scale group per lane and 128-dim step, scaled inside the MFMA
    o.k = n * pos + (UE ? 16 : 32) * q;
    o.ks = n * pos + kKScales + (UE ? 0 : 4 * (q >> 1));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o.v[e] = (4 * q + e) * pos + kVCodes + 8 * n;
      o.vs[e] = o.v[e] - kVCodes - 8 * n + kVScales + 4 * (n >> 3);
    }
  }
  const auto r0 = tile_rsrc(a, ids, blk_lo, t0, L, h, bs_shift);
  const auto r1 = tile_rsrc(a, ids, blk_lo, t0 + 16, L, h, bs_shift);
  constexpr uint32_t k2 = UE ? 64 : 16;  // offset of the lane's second 16 code bytes
  c.kc[0][0] = __builtin_amdgcn_raw_buffer_load_b128(r0, o.k, 0, 0);
  c.kc[0][1] = __builtin_amdgcn_raw_buffer_load_b128(r0, o.k + k2, 0, 0);
  c.kc[1][0] = __builtin_amdgcn_raw_buffer_load_b128(r1, o.k, 0, 0);
  c.kc[1][1] = __builtin_amdgcn_raw_buffer_load_b128(r1, o.k + k2, 0, 0);
  if constexpr (UE) {
    const i32x2 s0 = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r0, o.ks, 0, 0));
    const i32x2 s1 = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r1, o.ks, 0, 0));
    c.ksw[0][0] = s0[0];
    c.ksw[0][1] = s0[1];
    c.ksw[1][0] = s1[0];
    c.ksw[1][1] = s1[1];
  } else {
    c.ksw[0][0] = __builtin_amdgcn_raw_buffer_load_b32(r0, o.ks, 0, 0);
    c.ksw[1][0] = __builtin_amdgcn_raw_buffer_load_b32(r1, o.ks, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c.vc[e] = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r0, o.v[e], 0, 0));
    c.vsw[e] = __builtin_amdgcn_raw_buffer_load_b32(r0, o.vs[e], 0, 0);
    c.vc[4 + e] = __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r1, o.v[e], 0, 0));
    c.vsw[4 + e] = __builtin_amdgcn_raw_buffer_load_b32(r1, o.vs[e], 0, 0);
  }
  return c;
}

// One unit of the FP4 decode for a whole workgroup (every wave calls it with the same
// arguments): the tile-groups part_first + k tg_step (k < n_tg) of sequence b (length L)
// for kv head h0, merged into partition part_first; the unit's other partitions in
// [part_first, p_end) are written as empty.  Wave w (part) streams tokens [64 w, 64 w + 64)
// of each tile-group.  (The code keeps a head index hw: covering both heads of a token row
// with one workgroup, whole 544-byte rows, measured slower on MI355X: 52.4 vs 50.6 us at
// QG 16, as did balanced slices of 8 waves per CU, 52.4 us.  So did a work queue:
// persistent workgroups on a head pair taking 128-token items from a device counter, one
// barrier and one block-table read per item, 68 us per step against 54 us for these
// static runs; the same items dealt statically, 71 us.)
template <typename QT, bool UE>
__device__ __forceinline__ void fp4_unit(const DecodeArgs& a, const int lane, const int wave,
                                         const int b, const int h0, const int L,
                                         const int part_first, const int p_end,
                                         const int n_tg, const int tg_step) {
  constexpr int HPW = 1;            // kv heads per workgroup
  constexpr int W = kW;             // waves per workgroup
  constexpr int WPH = W / HPW;      // waves per head
  constexpr int TPW = 256 / WPH;    // tokens of a tile-group per wave
  constexpr int SPT = TPW / 32;     // 32-token steps per tile-group per wave
  constexpr int RPW = 16 / WPH;     // query rows a wave rotates
  constexpr int kQStride = kD + 8;        // f16 query row (halves)
  constexpr int kQBStride = 2 * kD + 16;  // e4m3 hi row then lo row (bytes)
  constexpr int kQBytes = HPW * 16 * (UE ? kQBStride : 2 * kQStride);
  // the merge: waves part > 0 leave their scaled accumulators, lane-major (16 KB each)
  constexpr int kMergeBytes = HPW * (WPH - 1) * 16 * 64 * 16;
  constexpr int kLdsBytes = kQBytes > kMergeBytes ? kQBytes : kMergeBytes;
  // Rotated query during the stream; the merge states after a barrier (same bytes).
  __shared__ __attribute__((aligned(16))) uint8_t lds_buf[kLdsBytes];
  __shared__ float lds_fac[HPW][16];
  __shared__ float lds_m[W][16];
  __shared__ float lds_l[W][16];

  const int hw = wave / WPH, part = wave % WPH;
  const int h = h0 + hw;
  const int p = part_first;
  _Float16* lds_q = reinterpret_cast<_Float16*>(lds_buf) + hw * 16 * kQStride;
  uint8_t* lds_qb = lds_buf + hw * 16 * kQBStride;

  // The query rows this wave rotates (rows [RPW part, RPW part + RPW) of head h, four at a
  // time, lane: row + lane / 16, dims 16 c .. 16 c + 15) and the rotation signs are loaded
  // before the block-table window: the rotation, which waits only for them (vector loads
  // return in order), runs under the first KV step's loads.
  const int NR = a.QL * a.QG;
  constexpr int kQW = sizeof(QT) == 4 ? 4 : 2;  // 16-byte words of a lane's 16 dims
  i32x4 q_raw[RPW / 4][kQW];
  i32x4 sg_raw = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int rp = 0; rp < RPW; rp += 4) {
    const int row = RPW * part + rp + (lane >> 4);
#pragma unroll
    for (int k = 0; k < kQW; ++k) q_raw[rp / 4][k] = i32x4{0, 0, 0, 0};
    if (row < NR) {
      const QT* src = reinterpret_cast<const QT*>(a.q) + ((int64_t)b * a.QL + row / a.QG) * a.q_ss +
                      (int64_t)(h * a.QG + row % a.QG) * a.q_sh + 16 * (lane & 15);
#pragma unroll
      for (int k = 0; k < kQW; ++k)
        q_raw[rp / 4][k] = *reinterpret_cast<const i32x4*>(src + k * (16 / (int)sizeof(QT)));
    }
  }
  {
    // through a buffer resource with no records when there are no signs (the load then
    // returns zeros): no branch, so no copy at a join that would wait for the query loads
    // before the block-table window is even requested
    const uint64_t base = (uint64_t)(a.rot_signs ? (const void*)a.rot_signs : a.q);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, a.rot_signs ? kD : 0,
        0x00020000);
    sg_raw = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (lane & 15), 0, 0);
  }


  const int n = lane & 15;   // unit row of the QK / softmax layout; PV column group
  const int q = lane >> 4;   // lane row group
  // unit rows r = j * QG + g: query row j (of QL per sequence), head g; query row j sees
  // the tokens t < L - QL + 1 + j (the causal window of its row)
  const int L_row = L - a.QL + 1 + (n < NR ? n / a.QG : 0);

  // ---- the stream.  Wave (hw, part) takes tokens [TPW part, TPW part + TPW) of each of
  //      the workgroup's tile-groups.  The first step's loads go out before the query
  //      rotation, so the rotation runs under their latency.
  const int bs_shift = 31 - __builtin_clz(a.block_size);
  // The wave's stream: 32-token steps c = 0, 1, ... ; step c covers tokens
  // [s_k + 32 (c % SPT), + 32) of tile-group k = c / SPT, s_k = 256 tg_k + TPW part.  Steps
  // holding tokens form a prefix.  Block ids of a window of tile-groups are preloaded
  // (lane i: tile-group kw + i / bpw, block i % bpw of its TPW tokens, clamped to the last
  // visible block so that no table entry past the sequence is read).
  const int bpw = TPW / a.block_size > 0 ? TPW / a.block_size : 1;
  const int win_tgs = 64 / bpw;
  int ids = 0, kw = -win_tgs;
  auto s_of = [&](int k) { return (part_first + k * tg_step) * kTileGroup + TPW * part; };
  auto load_ids = [&](int k0) {
    kw = k0;
    const int k = k0 + lane / bpw;
    int v = 0;
    if (k < n_tg) {
      const int sk = s_of(k);
      if (sk < L) {
        int bi = (sk >> bs_shift) + lane % bpw;
        const int blk_last = (L - 1) >> bs_shift;
        bi = bi > blk_last ? blk_last : bi;
        v = a.bt[(int64_t)b * a.bt_stride + bi];
      }
    }
    ids = v;
  };
  auto step_t0 = [&](int c) { return s_of(c / SPT) + 32 * (c % SPT); };
  auto step_ok = [&](int c) { return c < SPT * n_tg && step_t0(c) < L; };
  auto load_step = [&](int c, Chunk& dst) {
    const int k = c / SPT;
    if (k >= kw + win_tgs) load_ids(k);
    const int sk = s_of(k);
    dst = load_chunk<UE>(a, n, q, ids, (sk >> bs_shift) - (k - kw) * bpw, step_t0(c), L, h,
                         bs_shift);
  };
  // the first step's KV loads as soon as its block ids are in; the rotation below runs
  // under their latency (its query words were loaded before them)
  Chunk cA, cB;
  if (step_ok(0)) load_step(0, cA);


  // ---- rotated query of head h: wave (hw, part) takes rows [RPW part, RPW part + RPW),
  //      four at a time, lane (row + lane/16, dims 16 c .. 16 c + 15)
#pragma unroll
  for (int rp = 0; rp < RPW; rp += 4) {
    const int row = RPW * part + rp + (lane >> 4);
    const int c = lane & 15;
    float x[16];
    if constexpr (sizeof(QT) == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * k + e] = bits_f((uint32_t)q_raw[rp / 4][k][e]);
    } else {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const i32x4 v = q_raw[rp / 4][k];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[8 * k + 2 * e] = bf16_to_f((uint32_t)v[e] & 0xFFFFu);
          x[8 * k + 2 * e + 1] = bf16_to_f((uint32_t)v[e] >> 16);
        }
      }
    }
    if (a.rot_signs) {
      const i32x4 sg = sg_raw;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s8 = (int)(int8_t)((uint32_t)sg[e >> 2] >> (8 * (e & 3)));
        x[e] = s8 < 0 ? -x[e] : x[e];
      }
      // butterflies of stride 1, 2, 4, 8: inside the lane
#pragma unroll
      for (int st = 1; st < 16; st <<= 1) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if ((e & st) == 0) {
            const float u = x[e], v = x[e + st];
            x[e] = u + v;
            x[e + st] = u - v;
          }
        }
      }
      // strides 16, 32, 64, 128: partner lane c ^ 1, 2, 4, 8 of the same 16-lane row
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        const bool upper = (c & m) != 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float o = __shfl_xor(x[e], m, 64);
          x[e] = upper ? o - x[e] : x[e] + o;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] *= 0.0625f;  // 1 / sqrt(256)
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    if constexpr (!UE) {
      // f16: 2^sh puts amax in [2^14, 2^15)
      int sh = 0;
      if (amax > 0.f) {
        const int E = (int)((f_bits(amax) >> 23) & 0xFF) - 127;  // amax in [2^E, 2^(E+1))
        sh = 14 - (E < -126 ? -126 : E);
        sh = sh > 126 ? 126 : sh;
      }
      const float up = __builtin_ldexpf(1.f, sh);
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const f16x2 hv = f16x2{(_Float16)(x[2 * e] * up), (_Float16)(x[2 * e + 1] * up)};
        w[e] = __builtin_bit_cast(uint32_t, hv);
      }
      uint8_t* dst = reinterpret_cast<uint8_t*>(lds_q + row * kQStride + 16 * c);
      *reinterpret_cast<i32x4*>(dst) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
      *reinterpret_cast<i32x4*>(dst + 16) = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
      if (c == 0) lds_fac[hw][row] = a.softmax_scale * kLog2e * __builtin_ldexpf(1.f, -sh);
    } else {
      // e4m3 hi + lo pair of q' s_q, s_q = 2^(7 - E) putting amax in [64, 128): the pair
      // carries about 8 significant bits (the scaled MFMA takes fp8 for the query)
      int E = 0;
      if (amax > 0.f) {
        E = (int)((f_bits(amax) >> 23) & 0xFF) - 126;  // amax in [2^(E-1), 2^E)
        E = E < -100 ? -100 : (E > 100 ? 100 : E);
      }
      const float s_q = __builtin_ldexpf(1.f, 7 - E);
      int hiw[4], low[4];
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) {
        const float y0 = x[4 * w4] * s_q, y1 = x[4 * w4 + 1] * s_q;
        const float y2 = x[4 * w4 + 2] * s_q, y3 = x[4 * w4 + 3] * s_q;
        int hv = cvt_pk_e4m3<false>(y0, y1, 0);
        hv = cvt_pk_e4m3<true>(y2, y3, hv);
        int lv = cvt_pk_e4m3<false>(y0 - e4m3_to_f<0>(hv), y1 - e4m3_to_f<1>(hv), 0);
        lv = cvt_pk_e4m3<true>(y2 - e4m3_to_f<2>(hv), y3 - e4m3_to_f<3>(hv), lv);
        hiw[w4] = hv;
        low[w4] = lv;
      }
      uint8_t* dst = lds_qb + row * kQBStride + 16 * c;
      *reinterpret_cast<i32x4*>(dst) = i32x4{hiw[0], hiw[1], hiw[2], hiw[3]};
      *reinterpret_cast<i32x4*>(dst + kD) = i32x4{low[0], low[1], low[2], low[3]};
      if (c == 0) lds_fac[hw][row] = a.softmax_scale * kLog2e / s_q;
    }
  }
  __syncthreads();

  // B operand of QK is read from LDS at each use: f16 head n, dims 64 q + 8 kk .. + 8
  // (e4m3 scales), or e4m3 hi/lo bytes of head n from dim 16 q on (UE8M0 scales)
  const _Float16* qrow = lds_q + n * kQStride + 64 * q;
  const uint8_t* qbrow = lds_qb + n * kQBStride + 16 * q;
  const float fac = lds_fac[hw][n];

  float m_run = -INFINITY;  // reference of head n (exp2 units); acc/l are relative to it
  float l_run = 0.f;        // this lane's share of sum p for head n
  f32x4 acc[16];            // acc[mm][jj] = O[head 4q + jj][dim 16 n + mm]
#pragma unroll
  for (int mm = 0; mm < 16; ++mm) acc[mm] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one 32-token step: QK, online softmax, PV
  auto step = [&](const Chunk& cur, const int t0) {
      const auto& kc = cur.kc;
      const auto& ksw = cur.ksw;
      const auto& vc = cur.vc;
      const auto& vsw = cur.vsw;

      // ---- QK: s[T][jj] = score of token t0 + 16 T + 4 q + jj, head n
      f32x4 s[2];
#pragma unroll
      for (int T = 0; T < 2; ++T) {
        f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
        if constexpr (!UE) {
          const f16x2 s0 = splat_h(e4m3_byte(ksw[T][0], 2 * (q & 1)));
          const f16x2 s1 = splat_h(e4m3_byte(ksw[T][0], 2 * (q & 1) + 1));
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const uint32_t wd = (uint32_t)kc[T][kk >> 2][kk & 3];
            const f16x2 sc = kk < 4 ? s0 : s1;
            const f16x8 A = cat4(fp4_pair<0>(wd) * sc, fp4_pair<1>(wd) * sc,
                                 fp4_pair<2>(wd) * sc, fp4_pair<3>(wd) * sc);
            const f16x8 qb = *reinterpret_cast<const f16x8*>(qrow + 8 * kk);
            c4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb, c4, 0, 0, 0);
          }
        } else {
          // scaled fp4 x fp8 MFMA per 128-dim step s: A = this lane's 32 K codes (its
          // 32-dim group 4s + q of token n) with that group's UE8M0 byte as the block
          // scale; B = the query's e4m3 hi, then lo, in the matching k order (bytes
          // [16q, +16) and [64 + 16q, +16) of the step's 128 dims)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int scale = (int)((ksw[T][st] >> (8 * q)) & 0xFFu);
            const i32x4 kv = kc[T][st];
            const i32x8 A = {kv[0], kv[1], kv[2], kv[3], 0, 0, 0, 0};
#pragma unroll
            for (int part = 0; part < 2; ++part) {  // hi, lo
              const uint8_t* qb = qbrow + part * kD + 128 * st;
              const i32x4 b0 = *reinterpret_cast<const i32x4*>(qb);
              const i32x4 b1 = *reinterpret_cast<const i32x4*>(qb + 64);
              const i32x8 Bq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
              c4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, Bq, c4, 4, 0, 0, scale, 0,
                                                                     127);
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int t = t0 + 16 * T + 4 * q + jj;
          c4[jj] = t < L_row ? c4[jj] * fac : -INFINITY;
        }
        s[T] = c4;
      }

      __builtin_amdgcn_sched_barrier(0);
      // ---- online softmax (reference moves only when a score exceeds it)
      float mloc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      if (__builtin_amdgcn_ballot_w64(mloc > m_run)) {
        const float m_new = fmaxf(m_run, max_across_rows(mloc));
        // 0 while m_run = -inf; 1 for a row that has seen no token yet (both -inf)
        const float alpha = m_run == m_new ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
        // accumulator rows are heads 4q + jj: their factors live in lanes 4q + jj
        float al[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) al[jj] = __shfl(alpha, 4 * q + jj, 64);
#pragma unroll
        for (int mm = 0; mm < 16; ++mm)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[mm][jj] *= al[jj];
      }
      // a row that has seen no token (m_run = -inf) has only -inf scores: weight 0
      const float m_ref = m_run == -INFINITY ? 0.f : m_run;
      float pv[8];
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pv[4 * T + jj] = fast_exp2(s[T][jj] - m_ref);
#pragma unroll
      for (int e = 0; e < 8; ++e) l_run += pv[e];
      // A operand of PV: head n, k-slot 8q + e <-> token t0 + (e < 4 ? 4q + e : 16 + 4q + e - 4)
      const f16x8 pa = f16x8{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3],
                             (_Float16)pv[4], (_Float16)pv[5], (_Float16)pv[6], (_Float16)pv[7]};

      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!UE) {
      // ---- PV.  Token pair u = (2u, 2u+1); X / Y hold per byte the even / odd dim of the
      //      byte's position for both tokens (low nibble: token 2u).
      f16x2 vs[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int sb = (n >> 1) & 3;
        vs[u] = f16x2{(_Float16)e4m3_byte(vsw[2 * u], sb), (_Float16)e4m3_byte(vsw[2 * u + 1], sb)};
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t X[4], Y[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t wa = (uint32_t)vc[2 * u][hh], wb = (uint32_t)vc[2 * u + 1][hh];
          X[u] = (wa & 0x0F0F0F0Fu) | ((wb << 4) & 0xF0F0F0F0u);
          Y[u] = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);
        }
#define UQ_PV_BYTE(KB)                                                                         \
  {                                                                                            \
    const f16x8 bx = cat4(fp4_pair<KB>(X[0]) * vs[0], fp4_pair<KB>(X[1]) * vs[1],              \
                          fp4_pair<KB>(X[2]) * vs[2], fp4_pair<KB>(X[3]) * vs[3]);             \
    acc[8 * hh + 2 * KB] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bx, acc[8 * hh + 2 * KB], \
                                                                  0, 0, 0);                    \
    const f16x8 by = cat4(fp4_pair<KB>(Y[0]) * vs[0], fp4_pair<KB>(Y[1]) * vs[1],              \
                          fp4_pair<KB>(Y[2]) * vs[2], fp4_pair<KB>(Y[3]) * vs[3]);             \
    acc[8 * hh + 2 * KB + 1] =                                                                 \
        __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, by, acc[8 * hh + 2 * KB + 1], 0, 0, 0);      \
  }
        UQ_PV_BYTE(0)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BYTE(1)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BYTE(2)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BYTE(3)
        __builtin_amdgcn_sched_barrier(0);
#undef UQ_PV_BYTE
      }
      } else {
        // ---- PV in bf16 (a UE8M0 scale can leave the f16 range).  Each token's bytes are
        //      converted with its own power-of-two scale (exactly the operand of
        //      v_cvt_scalef32_pk_bf16_fp4; a scale byte of 0 gives 0), then v_perm pairs
        //      tokens 2u, 2u+1 per B register.
        typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, i32x4{(int)pack_bf16x2(pv[0], pv[1]), (int)pack_bf16x2(pv[2], pv[3]),
                          (int)pack_bf16x2(pv[4], pv[5]), (int)pack_bf16x2(pv[6], pv[7])});
        float vsc[8];
        uint32_t vcw[8][2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t eb = (vsw[e] >> (8 * ((n >> 1) & 3))) & 0xFFu;
          vsc[e] = bits_f(eb << 23);
          vcw[e][0] = eb ? (uint32_t)vc[e][0] : 0u;
          vcw[e][1] = eb ? (uint32_t)vc[e][1] : 0u;
        }
#define UQ_PV_BF(HH, KB)                                                                      \
  {                                                                                           \
    uint32_t cv[8];                                                                           \
    _Pragma("unroll") for (int e = 0; e < 8; ++e) cv[e] = __builtin_bit_cast(                 \
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(vcw[e][HH], vsc[e], KB));         \
    const bf16x8 bx = __builtin_bit_cast(                                                     \
        bf16x8, i32x4{(int)__builtin_amdgcn_perm(cv[1], cv[0], 0x05040100u),                   \
                      (int)__builtin_amdgcn_perm(cv[3], cv[2], 0x05040100u),                   \
                      (int)__builtin_amdgcn_perm(cv[5], cv[4], 0x05040100u),                   \
                      (int)__builtin_amdgcn_perm(cv[7], cv[6], 0x05040100u)});                 \
    const bf16x8 by = __builtin_bit_cast(                                                     \
        bf16x8, i32x4{(int)__builtin_amdgcn_perm(cv[1], cv[0], 0x07060302u),                   \
                      (int)__builtin_amdgcn_perm(cv[3], cv[2], 0x07060302u),                   \
                      (int)__builtin_amdgcn_perm(cv[5], cv[4], 0x07060302u),                   \
                      (int)__builtin_amdgcn_perm(cv[7], cv[6], 0x07060302u)});                 \
    acc[8 * HH + 2 * KB] =                                                                    \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, bx, acc[8 * HH + 2 * KB], 0, 0, 0);       \
    acc[8 * HH + 2 * KB + 1] =                                                                \
        __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, by, acc[8 * HH + 2 * KB + 1], 0, 0, 0);   \
  }
        UQ_PV_BF(0, 0)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BF(0, 1)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BF(0, 2)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BF(0, 3)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BF(1, 0)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BF(1, 1)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BF(1, 2)
        __builtin_amdgcn_sched_barrier(0);
        UQ_PV_BF(1, 3)
        __builtin_amdgcn_sched_barrier(0);
#undef UQ_PV_BF
      }
  };
  // two step buffers, alternating: the next step's loads are issued before this step
  if (step_ok(0)) {
    for (int c = 0;; c += 2) {
      const bool ok1 = step_ok(c + 1);
      if (ok1) load_step(c + 1, cB);
      step(cA, step_t0(c));
      if (!ok1) break;
      const bool ok2 = step_ok(c + 2);
      if (ok2) load_step(c + 2, cA);
      step(cB, step_t0(c + 1));
      if (!ok2) break;
    }
  }

  // ---- merge the WPH waves of each head: (m, l) per row, then the scaled accumulators.
  //      Waves part > 0 leave acc * factor in LDS, lane-major (conflict-free 16-byte
  //      accesses, the same lane layout on both sides); wave part 0 adds them to its own
  //      and writes the rows.
  const float l_tot = sum_across_rows(l_run);
  __syncthreads();  // every wave is done with the rotated query (the same LDS bytes)
  if (q == 0) {
    lds_m[wave][n] = m_run;
    lds_l[wave][n] = l_tot;
  }
  __syncthreads();
  f32x4 fs;  // this wave's factor for rows 4q .. 4q + 3
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int hd = 4 * q + jj;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WPH; ++w) M = fmaxf(M, lds_m[hw * WPH + w][hd]);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < WPH; ++w) {
      const float mw = lds_m[hw * WPH + w][hd];
      lsum += mw == -INFINITY ? 0.f : lds_l[hw * WPH + w][hd] * fast_exp2(mw - M);
    }
    const float ms = lds_m[wave][hd];
    fs[jj] = (ms == -INFINITY || !(lsum > 0.f)) ? 0.f : fast_exp2(ms - M) / lsum;
    if (part == 0 && n == 0 && hd < NR) {
      const int64_t row = (((int64_t)b * a.Hk + h) * a.P + p) * NR + hd;
      a.part_m[row] = M * kLn2;
      a.part_l[row] = lsum;
      // the run's other partitions: empty states
      for (int pe = part_first + 1; pe < p_end; ++pe) {
        a.part_m[row + (int64_t)(pe - p) * NR] = -INFINITY;
        a.part_l[row + (int64_t)(pe - p) * NR] = 0.f;
      }
    }
  }
  f32x4* st = reinterpret_cast<f32x4*>(lds_buf);
  if constexpr (WPH > 1) {
    if (part > 0) {
      f32x4* mine = st + (hw * (WPH - 1) + part - 1) * 16 * 64;
#pragma unroll
      for (int mm = 0; mm < 16; ++mm) mine[mm * 64 + lane] = acc[mm] * fs;
    }
    __syncthreads();
  }
  if (part == 0) {
    // acc[mm][jj] = O[row 4q + jj][dim 16n + mm]
#pragma unroll
    for (int mm = 0; mm < 16; ++mm) {
      f32x4 o = acc[mm] * fs;
#pragma unroll
      for (int w = 1; w < WPH; ++w) o += st[((hw * (WPH - 1) + w - 1) * 16 + mm) * 64 + lane];
      acc[mm] = o;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int row = 4 * q + jj;
      if (row < NR) {
        const int64_t prow = (((int64_t)b * a.Hk + h) * a.P + p) * NR + row;
        uint16_t* dst = a.part_o + prow * kD + 16 * n;
        i32x4 w0, w1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w0[e] = (int)pack_bf16x2(acc[2 * e][jj], acc[2 * e + 1][jj]);
          w1[e] = (int)pack_bf16x2(acc[8 + 2 * e][jj], acc[8 + 2 * e + 1][jj]);
        }
        *reinterpret_cast<i32x4*>(dst) = w0;
        *reinterpret_cast<i32x4*>(dst + 8) = w1;
      }
    }
  }

}

template <typename QT, bool UE>
__global__ __launch_bounds__(64 * kW, 2) void decode_fp4_kernel(DecodeArgs a) {
  constexpr int HPW = 1;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  {
    // workgroup = (kv head, sequence b, group grp), kv head fastest.  The kv heads of one
    // (sequence, group) share cache lines (a 272-byte slot is not line aligned), so they
    // are placed on one XCD -- workgroups are dealt to the 8 XCDs round robin, so the heads
    // go 8 apart in launch order -- and read the shared lines through one L2 (measured on
    // MI355X: HBM reads 1.42x -> 1.01x the slot bytes, 8 % faster).  The grid is padded to
    // a multiple of 8 Hk, which makes the map a bijection; the padding workgroups exit
    // here.
    const int NHG = a.Hk / HPW;
    const int64_t unit0 = blockIdx.x;
    const int64_t xc = unit0 % 8, j = unit0 / 8;
    const int64_t unit_id = ((j / NHG) * 8 + xc) * NHG + j % NHG;
    if (unit_id >= (int64_t)a.B * NHG * a.runs) return;  // workgroup-uniform, before any barrier
    const int b = (int)((unit_id / NHG) % a.B);
    const int grp = (int)(unit_id / ((int64_t)NHG * a.B));

    int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
    L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
    const int ntg = (L + kTileGroup - 1) / kTileGroup;
    // Partitions with tokens: p < pmax.  With one tile-group per partition the workgroup
    // owns the run of partitions [part_first, part_first + R) (R = run_len) and merges
    // them into partition part_first (the others are written as empty); otherwise it owns
    // partition part_first and its strided tile-groups p, p + P, ...
    const int pmax = a.P < ntg ? a.P : ntg;
    const int R = a.run_len > 0 ? a.run_len : 1;
    int part_first, p_end, n_tg, tg_step;
    if (a.run_len > 0) {
      // this sequence's pmax partitions in G nearly equal runs of at most R
      const int G = (pmax + R - 1) / R;
      if (grp >= G) return;  // workgroup-uniform: nothing written, never read
      part_first = (int)((int64_t)grp * pmax / G);
      p_end = (int)((int64_t)(grp + 1) * pmax / G);
      n_tg = p_end - part_first;
      tg_step = 1;
    } else {
      part_first = grp;
      if (part_first >= pmax) return;  // workgroup-uniform: nothing written, never read
      p_end = part_first + 1;
      n_tg = (ntg - part_first + a.P - 1) / a.P;
      n_tg = n_tg < a.TGPP ? n_tg : a.TGPP;
      tg_step = a.P;
    }

    fp4_unit<QT, UE>(a, lane, wave, b, (int)(unit_id % NHG) * HPW, L, part_first, p_end, n_tg,
                     tg_step);
  }
}

}  // namespace

hipError_t launch_decode_fp4(const DecodeArgs& a, bool q_is_f32, bool ue8m0, hipStream_t stream) {
  const int64_t units = (int64_t)a.B * a.Hk * a.runs;  // runs: workgroups per (b, h)
  if (units <= 0) return hipSuccess;
  // padded to a multiple of 8 Hk for the XCD placement of the kv heads (see the kernel)
  const int64_t pad = 8 * (int64_t)a.Hk;
  const int64_t wgs = (units + pad - 1) / pad * pad;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs), block(64 * kW);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, block, 0, stream, a); };
  if (ue8m0) {
    if (q_is_f32) go(decode_fp4_kernel<float, true>); else go(decode_fp4_kernel<uint16_t, true>);
  } else {
    if (q_is_f32) go(decode_fp4_kernel<float, false>); else go(decode_fp4_kernel<uint16_t, false>);
  }
  return hipGetLastError();
}

}  // namespace uq

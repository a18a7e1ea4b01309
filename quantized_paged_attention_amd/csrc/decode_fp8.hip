// decode_fp8.hip -- paged decode over a per-tensor-scaled OCP e4m3 cache, D = 128,
// GQA groups of up to 8 query heads, for gfx950.
//
// What is computed (ROCm/FlyDSL PR #825 "pa_decode_tile": per-tensor fp8 K/V decode with
// a cross-workgroup partition split; vLLM "ultraquant_decode_hd256" page: strided
// partition -> 256-token tile-group map, online softmax of STEP F, epilogue of STEP G):
// for a work unit (sequence b, kv head h, partition p) the softmax statistics
// (m, l, o = v_scale * sum exp(s - m) v / l) of the tokens of tile-groups p, p+P, ...
//
// Design (one 64-lane wave per work unit, no LDS):
//   * QK: one 16x16x128 fp8 MFMA per 16-token tile.  A = K codes straight from HBM
//     (lane = token, 32 head dims per lane), B = the query group as an e4m3 hi + lo pair:
//     columns 0-7 carry hi(q * s_q), columns 8-15 carry lo = q * s_q - hi, so one MFMA
//     gives both halves and a DPP row rotate adds them.  s_q is a per-row power of two,
//     so the pair reproduces a bf16 query exactly.
//   * Softmax is register resident in the MFMA output layout (lane = query column,
//     4 tokens per lane); row max/sum cross lanes with xor 16 / xor 32 only.
//   * PV: P (scaled by 256 so its small values stay normal in e4m3) is again split into
//     hi/lo columns; V^T comes from registers: each lane loads 8 head dims of 4 tokens
//     per tile and a v_perm byte transpose turns them into the 16x16x32 fp8 A operand.
//     The output lane keeps one query column, so the online-softmax rescale needs no
//     cross-lane traffic.
//   * KV bytes are loaded once, non-temporal, with the next tile pairs in flight while
//     the current pair computes.
#include "uq_device.h"
#include "uq_kernels.h"

namespace uq {
namespace {

constexpr int kD = 128;
constexpr int kPipe = 2;  // tile pairs in flight ahead of the one being computed

struct Tile {
  i32x4 k0, k1;  // K bytes [16r, 16r+16) and [64+16r, 64+16r+16) of token n
  i32x2 v[4];    // V bytes [8n, 8n+8) of tokens 4r + j
};

__device__ __forceinline__ void load_tile(Tile& t, const uint8_t* base, bool valid, int k_off,
                                          int v_off, int pos_stride) {
  if (valid) {
    t.k0 = nt_load(reinterpret_cast<const i32x4*>(base + k_off));
    t.k1 = nt_load(reinterpret_cast<const i32x4*>(base + k_off + 64));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.v[j] = nt_load(reinterpret_cast<const i32x2*>(base + v_off + j * pos_stride));
  } else {
    t.k0 = i32x4{0, 0, 0, 0};
    t.k1 = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) t.v[j] = i32x2{0, 0};
  }
}

template <typename QT, int W>
__global__ __launch_bounds__(64 * W) void decode_fp8_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * W + (threadIdx.x >> 6);
  if (unit >= (int64_t)a.P * a.B * a.Hk) return;
  const int h = (int)(unit % a.Hk);
  const int b = (int)((unit / a.Hk) % a.B);
  const int p = (int)(unit / ((int64_t)a.Hk * a.B));

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int ntg = (L + kTileGroup - 1) / kTileGroup;
  if (p >= ntg) return;  // empty partition: nothing written, never read by the reduce
  int trips = (ntg - p + a.P - 1) / a.P;
  trips = trips < a.TGPP ? trips : a.TGPP;

  const int r = lane >> 4, n = lane & 15;
  const int g = n & 7;
  const bool lo_col = n >= 8;

  // ---- query operand: hi/lo e4m3 pair of q * s_q, B layout of the 16x16x128 MFMA.
  // Byte j of lane group r holds head dim d = j < 16 ? 16r + j : 64 + 16r + (j - 16).
  float x[32];
  const bool qvalid = g < a.QG;
  {
    const QT* qp = reinterpret_cast<const QT*>(a.q) + (int64_t)b * a.q_ss +
                   (int64_t)(h * a.QG + (qvalid ? g : 0)) * a.q_sh;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const QT* src = qp + half * 64 + 16 * r;
      if constexpr (sizeof(QT) == 4) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[half * 16 + 4 * c + e] = v[e];
        }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(src + 8 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[half * 16 + 8 * c + 2 * e] = bf16_to_f((uint32_t)v[e] & 0xFFFFu);
            x[half * 16 + 8 * c + 2 * e + 1] = bf16_to_f((uint32_t)v[e] >> 16);
          }
        }
      }
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, xor_lane(amax, 16));
  amax = fmaxf(amax, xor_lane(amax, 32));
  // s_q = 2^(7 - E) with amax = f 2^E, f in [0.5, 1): amax * s_q in [64, 128)
  int E = 0;
  if (amax > 0.f) {
    E = (int)((f_bits(amax) >> 23) & 0xFF) - 126;
    E = E < -100 ? -100 : E;
  }
  const float s_q = bits_f((uint32_t)(127 + 7 - E) << 23);
  const float k_scale = a.k_scale ? *a.k_scale : 1.f;
  const float v_scale = a.v_scale ? *a.v_scale : 1.f;
  const float qk_mul = a.softmax_scale * k_scale * kLog2e / s_q;

  i32x8 qop;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float y0 = x[4 * w] * s_q, y1 = x[4 * w + 1] * s_q, y2 = x[4 * w + 2] * s_q,
          y3 = x[4 * w + 3] * s_q;
    int hw = cvt_pk_e4m3<false>(y0, y1, 0);
    hw = cvt_pk_e4m3<true>(y2, y3, hw);
    int lw = cvt_pk_e4m3<false>(y0 - e4m3_to_f<0>(hw), y1 - e4m3_to_f<1>(hw), 0);
    lw = cvt_pk_e4m3<true>(y2 - e4m3_to_f<2>(hw), y3 - e4m3_to_f<3>(hw), lw);
    qop[w] = qvalid ? (lo_col ? lw : hw) : 0;
  }

  // ---- state
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int pos_stride = a.pos_stride;
  const int k_off = n * pos_stride + 16 * r;
  const int v_off = 4 * r * pos_stride + kD + 8 * n;
  const uint8_t* head_base = a.cache + (int64_t)h * a.slot_bytes;
  const int32_t* bt_row = a.bt + (int64_t)b * a.bt_stride;

  for (int it = 0; it < trips; ++it) {
    const int tg_start = (p + it * a.P) * kTileGroup;
    // block id of tile t held by lane t (tiles past the context are not looked up)
    int my_blk = 0;
    if (lane < 16 && tg_start + 16 * lane < L) my_blk = bt_row[(tg_start + 16 * lane) / a.block_size];

    auto tile_base = [&](int t) -> const uint8_t* {
      const int blk = __builtin_amdgcn_readlane(my_blk, t);
      const int tok = tg_start + 16 * t;
      return head_base + (int64_t)blk * a.blk_stride + (int64_t)(tok % a.block_size) * pos_stride;
    };

    Tile ring[kPipe + 1][2];
#pragma unroll
    for (int s = 0; s < kPipe; ++s) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int t = 2 * s + tt;
        const bool valid = tg_start + 16 * t < L;
        load_tile(ring[s][tt], valid ? tile_base(t) : head_base, valid, k_off, v_off, pos_stride);
      }
    }

#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      // issue the loads kPipe pairs ahead
      if (pr + kPipe < 8) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int t = 2 * (pr + kPipe) + tt;
          const bool valid = tg_start + 16 * t < L;
          load_tile(ring[(pr + kPipe) % (kPipe + 1)][tt], valid ? tile_base(t) : head_base,
                    valid, k_off, v_off, pos_stride);
        }
      }
      Tile* cur = ring[pr % (kPipe + 1)];
      const int pair_start = tg_start + 32 * pr;

      // ---- QK: S^T[token][column] for both tiles
      float s[2][4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const i32x8 kop = {cur[tt].k0[0], cur[tt].k0[1], cur[tt].k0[2], cur[tt].k0[3],
                           cur[tt].k1[0], cur[tt].k1[1], cur[tt].k1[2], cur[tt].k1[3]};
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qop, z, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v = z[j] + row_ror8(z[j]);  // hi column + lo column
          v *= qk_mul;
          const int tok = pair_start + 16 * tt + 4 * r + j;
          s[tt][j] = tok < L ? v : -INFINITY;
        }
      }
      // ---- online softmax (base 2)
      float mloc = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mloc = fmaxf(mloc, xor_lane(mloc, 16));
      mloc = fmaxf(mloc, xor_lane(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float pv[2][4];
      float psum = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[tt][j] = fast_exp2(s[tt][j] - m_use);
          psum += pv[tt][j];
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] *= alpha;

      // ---- P operand: e4m3 hi (columns 0-7) / lo (columns 8-15) of 256 p
      int pw[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const float y0 = pv[tt][0] * 256.f, y1 = pv[tt][1] * 256.f, y2 = pv[tt][2] * 256.f,
                    y3 = pv[tt][3] * 256.f;
        int hw = cvt_pk_e4m3<false>(y0, y1, 0);
        hw = cvt_pk_e4m3<true>(y2, y3, hw);
        int lw = cvt_pk_e4m3<false>(y0 - e4m3_to_f<0>(hw), y1 - e4m3_to_f<1>(hw), 0);
        lw = cvt_pk_e4m3<true>(y2 - e4m3_to_f<2>(hw), y3 - e4m3_to_f<3>(hw), lw);
        pw[tt] = lo_col ? lw : hw;
      }
      const long pop = (long)(uint32_t)pw[0] | ((long)(uint32_t)pw[1] << 32);

      // ---- V^T operand: byte transpose of 8 dims x 4 tokens per tile; masked tokens -> 0
      uint32_t vt[2][8];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        uint32_t lo4[4], hi4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool ok = pair_start + 16 * tt + 4 * r + j < L;
          lo4[j] = ok ? (uint32_t)cur[tt].v[j][0] : 0u;
          hi4[j] = ok ? (uint32_t)cur[tt].v[j][1] : 0u;
        }
        transpose4x4_bytes(lo4, &vt[tt][0]);
        transpose4x4_bytes(hi4, &vt[tt][4]);
      }
      // ---- PV: acc[m][j'] accumulates O^T[d = 32 r' + 8 j' + m][column n']
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const long vop = (long)vt[0][m] | ((long)vt[1][m] << 32);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(vop, pop, acc[m], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: add lo columns into hi columns, normalise, store bf16 partials
  float l_tot = l_run + xor_lane(l_run, 16);
  l_tot += xor_lane(l_tot, 32);
  const float inv = v_scale / (256.f * (l_tot > 0.f ? l_tot : 1.f));
  float o[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) o[m][j] = (acc[m][j] + row_ror8(acc[m][j])) * inv;
  if (n < a.QG) {
    const int64_t row = (((int64_t)b * a.Hk + h) * a.P + p) * a.QG + n;
    uint16_t* dst = a.part_o + row * kD + 32 * r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      i32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (int)pack_bf16x2(o[2 * e][j], o[2 * e + 1][j]);
      *reinterpret_cast<i32x4*>(dst + 8 * j) = w;
    }
    if (r == 0) {
      a.part_m[row] = m_run * kLn2;
      a.part_l[row] = l_tot;
    }
  }
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, bool q_is_f32, hipStream_t stream) {
  constexpr int W = 4;
  const int64_t units = (int64_t)a.P * a.B * a.Hk;
  const dim3 grid((unsigned)((units + W - 1) / W));
  if (q_is_f32)
    hipLaunchKernelGGL((decode_fp8_kernel<float, W>), grid, dim3(64 * W), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_fp8_kernel<uint16_t, W>), grid, dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uq

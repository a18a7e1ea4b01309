// index_score.hip -- nvfp4 index scores for gfx950.
//
// What is computed (vLLM "nvfp4_index_decode/kernel" page, compile_score_decode: page
// layout of load_tile, per-page reduction of frag_max / score_cgs, causal limit of the
// trailing query rows): for request r, query row j < QL, index head h and page
// b < ceil(L_r / 128), the maximum over the page's tokens t <= L_r - QL + j of
// q[r QL + j, h, :] . k[t, :], with k = e2m1(code) * e4m3(scale of its 16-dim group);
// -inf when the page holds no such token.
//
// Design: one wave per (request, page), four waves per workgroup (measured on MI355X:
// more pages per wave, with the next page loaded under the current one, lose to the
// extra waves in flight).  The code keeps the multi-page loop (kPagesPerWave).
//   * Every e2m1 * e4m3 product and every e4m3 query value is exact in f16, so the page
//     is dequantised exactly (one v_cvt_scalef32_pk_f16_fp4 with unit scale and one
//     packed f16 multiply per byte) and the dot products run on v_mfma_f32_16x16x32_f16
//     with exact products and fp32 accumulation.
//   * A = K tile (lane = token, 32 consecutive dims per lane), B = the request's query
//     rows (columns = (j, h), at most 32: two column tiles).  The output layout puts
//     4 tokens of one column in a lane; masked tokens are selected to -inf (never
//     multiplied, so garbage past the sequence cannot leak), the page max is kept per
//     lane and reduced across the four lane rows once per page.
//   * A whole page (8 tiles: 128 code bytes + 1 scale word per lane, non-temporal) is in
//     registers before its first MFMA; the query operands are converted once per wave.
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
constexpr int kPagesPerWave = 1;
constexpr int kPagesPerGroup = kWaves * kPagesPerWave;

template <int sel>
__device__ __forceinline__ f16x2 fp4_pair(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, sel);
}

__device__ __forceinline__ f16x8 cat4(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 e4m3 bytes (two words, low byte first) -> 8 f16 (exact)
__device__ __forceinline__ f16x8 e4m3x8_to_f16(int w0, int w1) {
  return f16x8{(_Float16)e4m3_to_f<0>(w0), (_Float16)e4m3_to_f<1>(w0),
               (_Float16)e4m3_to_f<2>(w0), (_Float16)e4m3_to_f<3>(w0),
               (_Float16)e4m3_to_f<0>(w1), (_Float16)e4m3_to_f<1>(w1),
               (_Float16)e4m3_to_f<2>(w1), (_Float16)e4m3_to_f<3>(w1)};
}

struct Page {
  i32x4 kc[8];       // codes [16 q, 16 q + 16) of tokens 16 T + n
  uint32_t ksw[8];   // the scale word of groups 2q, 2q + 1 of those tokens
};

__device__ __forceinline__ void load_page(const uint8_t* pg, int n, int q, Page& d) {
#pragma unroll
  for (int T = 0; T < 8; ++T) {
    const int t = 16 * T + n;
    d.kc[T] = nt_load(reinterpret_cast<const i32x4*>(pg + t * kCodeBytes + 16 * q));
    d.ksw[T] = nt_load(reinterpret_cast<const uint32_t*>(pg + kScaleRegion + t * kScaleBytes +
                                                         4 * (q >> 1)));
  }
}

__global__ __launch_bounds__(64 * kWaves) void index_score_kernel(IndexArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // workgroup = (request r, chunk of kPagesPerGroup pages); wave w scores pages
  // chunk_base + w, + kWaves, ... (kPagesPerWave of them)
  const int per_req = (a.max_blocks + kPagesPerGroup - 1) / kPagesPerGroup;
  const int r = blockIdx.x / per_req;
  const int b0 = (blockIdx.x % per_req) * kPagesPerGroup + wave;
  // The table entries are read together with the length (entries below max_blocks are
  // inside the table row; one past the sequence is read but never used).
  int pid = 0;
  if (lane < kPagesPerWave && b0 + kWaves * lane < a.max_blocks)
    pid = a.bt[(int64_t)r * a.bt_stride + b0 + kWaves * lane];
  const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[r]);
  int nblk = (L + kPageTokens - 1) / kPageTokens;
  nblk = nblk < a.max_blocks ? nblk : a.max_blocks;
  if (b0 >= nblk) return;  // cells of pages past the sequence are left untouched
  const int npg = (nblk - b0 + kWaves - 1) / kWaves < kPagesPerWave
                      ? (nblk - b0 + kWaves - 1) / kWaves : kPagesPerWave;

  const int n = lane & 15;  // token of a tile (A) / column of a tile (B, output)
  const int q = lane >> 4;  // dims 32q .. 32q + 31
  const int R = a.QL * a.H;

  // page ids of this wave's pages: lane i < npg holds page b0 + kWaves i
  auto page_ptr = [&](int i) {
    const int id = __builtin_amdgcn_readlane(pid, i);
    return a.pages + (int64_t)id * a.page_stride;
  };
  Page cur, nxt;
  load_page(page_ptr(0), n, q, cur);

  // ---- query rows: column c = j * H + h; B operand dims 32 q + 8 kk .. + 8
  const int ncol_tiles = R > 16 ? 2 : 1;
  f16x8 qb[2][4];
  int lim0[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int col = 16 * ct + n;
    lim0[ct] = -1;
    if (col < R && ct < ncol_tiles) {
      const int j = col / a.H, hh = col % a.H;
      lim0[ct] = L - a.QL + j;  // last visible token of row j
      const uint8_t* src = a.q + ((int64_t)r * a.QL + j) * a.q_st + (int64_t)hh * a.q_sh + 32 * q;
      const i32x4 w0 = *reinterpret_cast<const i32x4*>(src);
      const i32x4 w1 = *reinterpret_cast<const i32x4*>(src + 16);
      qb[ct][0] = e4m3x8_to_f16(w0[0], w0[1]);
      qb[ct][1] = e4m3x8_to_f16(w0[2], w0[3]);
      qb[ct][2] = e4m3x8_to_f16(w1[0], w1[1]);
      qb[ct][3] = e4m3x8_to_f16(w1[2], w1[3]);
    } else {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) qb[ct][kk] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  for (int i = 0; i < npg; ++i) {
    if (i + 1 < npg) load_page(page_ptr(i + 1), n, q, nxt);  // next page under this one
    const int b = b0 + kWaves * i;
    float best[2] = {-INFINITY, -INFINITY};
    const int t_page = b * kPageTokens;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const uint32_t sw = cur.ksw[T] >> (16 * (q & 1));
      const _Float16 s0h = (_Float16)e4m3_to_f<0>((int)sw), s1h = (_Float16)e4m3_to_f<1>((int)sw);
      const f16x2 s0 = f16x2{s0h, s0h}, s1 = f16x2{s1h, s1h};
      f16x8 A[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t wd = (uint32_t)cur.kc[T][kk];
        const f16x2 sc = kk < 2 ? s0 : s1;
        A[kk] = cat4(fp4_pair<0>(wd) * sc, fp4_pair<1>(wd) * sc, fp4_pair<2>(wd) * sc,
                     fp4_pair<3>(wd) * sc);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        if (ct < ncol_tiles) {
          f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            c4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[kk], qb[ct][kk], c4, 0, 0, 0);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int t = t_page + 16 * T + 4 * q + jj;
            best[ct] = fmaxf(best[ct], t <= lim0[ct] ? c4[jj] : -INFINITY);
          }
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      if (ct < ncol_tiles) {
        const float m = max_across_rows(best[ct]);
        const int col = 16 * ct + n;
        if (q == 0 && col < R) {
          const int j = col / a.H, hh = col % a.H;
          a.scores[(int64_t)hh * a.s_sh + ((int64_t)r * a.QL + j) * a.s_st + b] = m;
        }
      }
    }
    cur = nxt;
  }
}

}  // namespace

hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream) {
  const int64_t per_req = (a.max_blocks + kPagesPerGroup - 1) / kPagesPerGroup;
  const int64_t wgs = per_req * a.num_reqs;
  if (wgs <= 0) return hipSuccess;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(index_score_kernel, dim3((unsigned)wgs), dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace uq

// reduce.hip -- flash-combine of per-partition decode statistics (ROCm/FlyDSL PR #825
// "pa_decode_tile": cross-workgroup partition split merged by a parallel reduce kernel;
// its empty-partition fix: partitions without tokens must not contribute).
//
// For output row (sequence b, query head hq; with several query rows per sequence, query
// row j of b) with n = min(P, ceil(L / 256)) partitions,
// over the partitions with l_p > 0 (a partition without tokens, or one whose tokens the
// decode merged into a neighbouring partition's statistics, has l_p = 0):
//   M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p   (0 if none).
//
// Layout of the work: a 16-byte load covers 8 dims of one partial row, so one wave load
// reads 64 / (D / 8) whole partial rows (4 at D = 128, 2 at D = 256).  A row's partitions
// are shared by S waves of one workgroup (S chosen on the host so that there are enough
// waves to fill the chip when there are few rows and many partitions, while every wave
// keeps at least 64 of the partitions a row can have).  All (m, l) of a
// row are loaded at once (up to 512 partitions in registers), M and the denominator are
// reduced across the wave, the partitions with l > 0 are compacted into an LDS list
// (ballot + mbcnt), and the waves stream only those partial rows, 8 per lane in flight;
// the S partial sums meet in LDS.  So a row costs two dependent memory round trips.
#include "uq_device.h"
#include "uq_kernels.h"

namespace uq {
namespace {

template <int D, typename OT, int S, int kChunks>
__global__ __launch_bounds__(S <= 4 ? 256 : 64 * S) void reduce_kernel(ReduceArgs a) {
  constexpr int LPR = D / 8;       // lanes per partial row (16-byte loads)
  constexpr int G = 64 / LPR;      // partial rows per wave load
  constexpr int U = kChunks == 1 ? 4 : 8;  // partial rows in flight per lane
  // kChunks: (m, l) of up to 64 * kChunks partitions are held in registers
  constexpr int RPB = S == 1 ? 4 : 1;  // rows per workgroup
  __shared__ int lst_p[RPB][64 * kChunks];    // live partitions of the row, compacted
  __shared__ float lst_w[RPB][64 * kChunks];  // and their weights
  __shared__ int lst_n[RPB];
  __shared__ __attribute__((aligned(16))) float lds_acc[S > 1 ? S : 1][D];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = S == 1 ? (int64_t)blockIdx.x * 4 + wave : (int64_t)blockIdx.x;
  const int s = S == 1 ? 0 : wave;
  const int slot = S == 1 ? wave : 0;
  const int64_t rows = (int64_t)a.B * a.Hk * a.QG;
  if (S == 1 && row >= rows) return;  // (S > 1: one row per workgroup, grid = rows)
  const int g = (int)(row % a.QG);
  const int h = (int)((row / a.QG) % a.Hk);
  const int b = (int)(row / ((int64_t)a.QG * a.Hk));

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int ntg = (L + kTileGroup - 1) / kTileGroup;
  const int n = ntg < a.P ? ntg : a.P;
  const int64_t ml0 = ((int64_t)b * a.Hk + h) * a.P * a.QG + g;  // + p * QG
  const int pg = lane / LPR, dl = lane % LPR;
  const uint16_t* o0 = a.part_o + ml0 * D + 8 * dl;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float M = -INFINITY, den = 0.f;

  if (n <= 64 * kChunks) {
    // (m, l) of every partition at once: lane p of chunk c holds partition 64 c + p.
    // Through buffer resources whose record count ends at partition n: the loads past it
    // return zero with no branch, so all of them are in flight together (a conditional
    // load per chunk left a copy at each join that waited for it: one round trip per
    // chunk and statistic).
    auto stat_rsrc = [&](const float* base) {
      const uint64_t ad = (uint64_t)(base + ml0);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)ad);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(ad >> 32));
      return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                               (short)0, __builtin_amdgcn_readfirstlane(n * a.QG * 4),
                                               0x00020000);
    };
    const auto rl = stat_rsrc(a.part_l), rm = stat_rsrc(a.part_m);
    float mv[kChunks], lv[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const uint32_t off = (uint32_t)((64 * c + lane) * a.QG * 4);
      lv[c] = bits_f((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rl, off, 0, 0));
      mv[c] = bits_f((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rm, off, 0, 0));
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) M = fmaxf(M, lv[c] > 0.f ? mv[c] : -INFINITY);
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) M = fmaxf(M, xor_lane(M, sh));
    float wv[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      wv[c] = lv[c] > 0.f ? lv[c] * __expf(mv[c] - M) : 0.f;
      den += wv[c];
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) den += xor_lane(den, sh);
    // compact the partitions with l > 0 (merged-away and empty ones drop out)
    if (S == 1 || s == 0) {
      int base = 0;
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const bool live = wv[c] > 0.f;
        const uint64_t mask = __builtin_amdgcn_ballot_w64(live);
        if (live) {
          const int rank = __builtin_amdgcn_mbcnt_hi(
              (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
          lst_p[slot][base + rank] = 64 * c + lane;
          lst_w[slot][base + rank] = wv[c];
        }
        base += __builtin_popcountll(mask);
      }
      if (lane == 0) lst_n[slot] = base;
    }
    if constexpr (S > 1) {
      __syncthreads();
    } else {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
    }
    const int count = lst_n[slot];
    // this wave's share of the live list: entries s + S (pg + G i)
    constexpr int kStep = S * G;
    for (int j0 = s + S * pg; j0 < count; j0 += U * kStep) {
      float w[U];
      int pp[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * kStep;
        const bool ok = j < count;
        pp[u] = ok ? lst_p[slot][j] : 0;
        w[u] = ok ? lst_w[slot][j] : 0.f;
      }
      i32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        raw[u] = i32x4{0, 0, 0, 0};
        if (w[u] > 0.f) raw[u] = *reinterpret_cast<const i32x4*>(o0 + (int64_t)pp[u] * a.QG * D);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w[u] * bf16_to_f((uint32_t)raw[u][e] & 0xFFFFu);
          acc[2 * e + 1] += w[u] * bf16_to_f((uint32_t)raw[u][e] >> 16);
        }
    }
  } else {
    // many partitions: one online pass for (M, den), then (m, l) and rows in batches
    for (int p = lane; p < n; p += 64) {
      const int64_t ml = ml0 + (int64_t)p * a.QG;
      const float l = a.part_l[ml];
      if (!(l > 0.f)) continue;
      const float m = a.part_m[ml];
      const float Mn = fmaxf(M, m);
      den = den * __expf(M - Mn) + l * __expf(m - Mn);  // M = -inf only while den = 0
      M = Mn;
    }
    {
      float Mw = M;
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) Mw = fmaxf(Mw, xor_lane(Mw, sh));
      den = M == -INFINITY ? 0.f : den * __expf(M - Mw);
      M = Mw;
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) den += xor_lane(den, sh);
    constexpr int kStep = S * G;
    for (int p = s + S * pg; p < n; p += U * kStep) {
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pp = p + u * kStep;
        float wl = 0.f;
        if (pp < n) {
          const int64_t ml = ml0 + (int64_t)pp * a.QG;
          const float l = a.part_l[ml];
          wl = l > 0.f ? l * __expf(a.part_m[ml] - M) : 0.f;
        }
        w[u] = wl;
      }
      i32x4 raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        raw[u] = i32x4{0, 0, 0, 0};
        if (w[u] > 0.f)
          raw[u] = *reinterpret_cast<const i32x4*>(o0 + (int64_t)(p + u * kStep) * a.QG * D);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w[u] * bf16_to_f((uint32_t)raw[u][e] & 0xFFFFu);
          acc[2 * e + 1] += w[u] * bf16_to_f((uint32_t)raw[u][e] >> 16);
        }
    }
  }

  // sum over the G partial rows of each wave load (lanes dl, dl + LPR, ...)
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (G == 4) {
      acc[e] = sum_across_rows(acc[e]);
    } else {
      auto t = __builtin_amdgcn_permlane32_swap(f_bits(acc[e]), f_bits(acc[e]), false, false);
      acc[e] = bits_f(t[0]) + bits_f(t[1]);
    }
  }
  if constexpr (S > 1) {
    if (pg == 0) {
      *reinterpret_cast<f32x4*>(&lds_acc[s][8 * dl]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4*>(&lds_acc[s][8 * dl + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
    __syncthreads();
    if (s != 0) return;
    if (pg == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = lds_acc[0][8 * dl + e];
      for (int w = 1; w < S; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += lds_acc[w][8 * dl + e];
    }
  }
  if (pg != 0) return;
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int qgh = a.QG / a.QL;  // query heads per kv head; row g = query g / qgh, head g % qgh
  OT* dst = reinterpret_cast<OT*>(a.out) + ((int64_t)b * a.QL + g / qgh) * a.o_ss +
            (int64_t)(h * qgh + g % qgh) * a.o_sh + 8 * dl;
  if constexpr (sizeof(OT) == 4) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]} * inv;
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]} * inv;
  } else {
    *reinterpret_cast<i32x4*>(dst) =
        i32x4{(int)pack_bf16x2(acc[0] * inv, acc[1] * inv), (int)pack_bf16x2(acc[2] * inv, acc[3] * inv),
              (int)pack_bf16x2(acc[4] * inv, acc[5] * inv), (int)pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  }
}

template <int D, typename OT, int C>
hipError_t launch_dc(const ReduceArgs& a, int64_t rows, hipStream_t stream) {
  // waves per row: the smallest S with rows * S >= 4096 waves, at most 16, and at least 64
  // partitions a row can have per wave (measured on MI355X: with 128 rows of 293
  // partitions, 4 waves per row take 8.5 us, 16 take 11.6 us; the cross-wave merge costs
  // more than the split gains once a wave has few partial rows)
  int64_t parts = ((int64_t)a.max_seq_len + 255) / 256;
  if (parts > a.P) parts = a.P;
  int S = 1;
  while (S < 16 && rows * S < 4096 && parts >= 128 * S) S *= 2;
  switch (S) {
    case 1:
      hipLaunchKernelGGL((reduce_kernel<D, OT, 1, C>), dim3((unsigned)((rows + 3) / 4)), dim3(256),
                         0, stream, a);
      break;
    case 2:
      hipLaunchKernelGGL((reduce_kernel<D, OT, 2, C>), dim3((unsigned)rows), dim3(128), 0, stream, a);
      break;
    case 4:
      hipLaunchKernelGGL((reduce_kernel<D, OT, 4, C>), dim3((unsigned)rows), dim3(256), 0, stream, a);
      break;
    case 8:
      hipLaunchKernelGGL((reduce_kernel<D, OT, 8, C>), dim3((unsigned)rows), dim3(512), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL((reduce_kernel<D, OT, 16, C>), dim3((unsigned)rows), dim3(1024), 0, stream,
                         a);
      break;
  }
  return hipGetLastError();
}

template <int D, typename OT>
hipError_t launch_d(const ReduceArgs& a, int64_t rows, hipStream_t stream) {
  // up to 64 partitions: one register chunk of statistics (fewer registers, more waves)
  return a.P <= 64 ? launch_dc<D, OT, 1>(a, rows, stream) : launch_dc<D, OT, 8>(a, rows, stream);
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, bool out_is_f32, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hk * a.QG;
  if (rows <= 0) return hipSuccess;
  if (rows > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (a.D == 128)
    return out_is_f32 ? launch_d<128, float>(a, rows, stream) : launch_d<128, uint16_t>(a, rows, stream);
  return out_is_f32 ? launch_d<256, float>(a, rows, stream) : launch_d<256, uint16_t>(a, rows, stream);
}

}  // namespace uq

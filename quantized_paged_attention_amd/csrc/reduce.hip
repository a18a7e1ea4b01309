// reduce.hip -- flash-combine of per-partition decode statistics (ROCm/FlyDSL PR #825
// "pa_decode_tile": cross-workgroup partition split merged by a parallel reduce kernel;
// its empty-partition fix: partitions without tokens must not contribute).
//
// One wave per output row (sequence b, query head hq).  Lane p of a 64-partition chunk
// loads (m_p, l_p) and forms w_p = l_p exp(m_p - M); the wave then streams the bf16
// partial rows, broadcasting w_p with readlane, eight partitions in flight at a time.
#include "uq_device.h"
#include "uq_kernels.h"

namespace uq {
namespace {

template <int D, typename OT>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  constexpr int E = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)a.B * a.Hk * a.QG;
  if (row >= rows) return;
  const int g = (int)(row % a.QG);
  const int h = (int)((row / a.QG) % a.Hk);
  const int b = (int)(row / ((int64_t)a.QG * a.Hk));

  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int ntg = (L + kTileGroup - 1) / kTileGroup;
  const int n = ntg < a.P ? ntg : a.P;

  const int64_t ml0 = ((int64_t)b * a.Hk + h) * a.P * a.QG + g;  // + p * QG
  // pass 1: M = max over the partitions that hold tokens
  float M = -INFINITY;
  for (int p = lane; p < n; p += 64) M = fmaxf(M, a.part_m[ml0 + (int64_t)p * a.QG]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, xor_lane(M, s));

  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float den = 0.f;
  const uint16_t* o0 = a.part_o + ml0 * D + lane * E;
  for (int c = 0; c < n; c += 64) {
    float w = 0.f;
    if (c + lane < n) {
      const int64_t ml = ml0 + (int64_t)(c + lane) * a.QG;
      w = a.part_l[ml] * __expf(a.part_m[ml] - M);
    }
    float wsum = w;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) wsum += xor_lane(wsum, s);
    den += wsum;
    const int cn = n - c < 64 ? n - c : 64;
    int k = 0;
    for (; k + 8 <= cn; k += 8) {
      uint32_t raw[8][E / 2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint16_t* src = o0 + (int64_t)(c + k + u) * a.QG * D;
        if constexpr (E == 2) {
          raw[u][0] = *reinterpret_cast<const uint32_t*>(src);
        } else {
          const i32x2 v = *reinterpret_cast<const i32x2*>(src);
          raw[u][0] = (uint32_t)v[0];
          raw[u][1] = (uint32_t)v[1];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = bits_f((uint32_t)__builtin_amdgcn_readlane((int)f_bits(w), k + u));
#pragma unroll
        for (int e = 0; e < E / 2; ++e) {
          acc[2 * e] += wu * bf16_to_f(raw[u][e] & 0xFFFFu);
          acc[2 * e + 1] += wu * bf16_to_f(raw[u][e] >> 16);
        }
      }
    }
    for (; k < cn; ++k) {
      const uint16_t* src = o0 + (int64_t)(c + k) * a.QG * D;
      const float wu = bits_f((uint32_t)__builtin_amdgcn_readlane((int)f_bits(w), k));
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += wu * bf16_to_f(src[e]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  OT* dst = reinterpret_cast<OT*>(a.out) + (int64_t)b * a.o_ss + (int64_t)(h * a.QG + g) * a.o_sh +
            lane * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float v = acc[e] * inv;
    if constexpr (sizeof(OT) == 4)
      dst[e] = v;
    else
      dst[e] = (OT)bf16_bits(v);
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, bool out_is_f32, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hk * a.QG;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (a.D == 128) {
    if (out_is_f32)
      hipLaunchKernelGGL((reduce_kernel<128, float>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((reduce_kernel<128, uint16_t>), grid, dim3(256), 0, stream, a);
  } else {
    if (out_is_f32)
      hipLaunchKernelGGL((reduce_kernel<256, float>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((reduce_kernel<256, uint16_t>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace uq

// uq_device.h -- small CDNA4 (gfx950) device helpers shared by the libuq kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "uq_kernels.h"

namespace uq {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Lane exchange across 16-lane rows / 32-lane halves (ds_bpermute based).
__device__ __forceinline__ float xor_lane(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reductions across the four 16-lane rows of a wave with the gfx950 lane-swap
// instructions (VALU, no LDS round trip): permlane16_swap(x, x) returns the values of the
// even and of the odd row of each row pair, permlane32_swap(x, x) those of the lower and
// the upper half, so combining the two halves of each result reduces over lanes
// l, l ^ 16, l ^ 32, l ^ 48.
__device__ __forceinline__ float max_across_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = fmaxf(bits_f(a[0]), bits_f(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return fmaxf(bits_f(b[0]), bits_f(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  x = bits_f(a[0]) + bits_f(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(b[0]) + bits_f(b[1]);
}

// Exchange with the lane n ^ 8 of the same 16-lane row (DPP row rotate by 8).  The DPP
// moves here read valid lanes only, so bound_ctrl changes no result; it lets the compiler
// fold the move into the VALU instruction that consumes it (one v_add_f32_dpp, say).
__device__ __forceinline__ float row_ror8(float v) {
  return bits_f((uint32_t)__builtin_amdgcn_mov_dpp((int)f_bits(v), 0x128, 0xF, 0xF, true));
}

// The four values of the lane's quad (lanes 4k .. 4k+3), each broadcast to every lane of
// the quad (DPP quad_perm [j, j, j, j] for j = 0..3).
__device__ __forceinline__ void quad_values(float v, float out[4]) {
  const int x = (int)f_bits(v);
  out[0] = bits_f((uint32_t)__builtin_amdgcn_mov_dpp(x, 0x00, 0xF, 0xF, true));
  out[1] = bits_f((uint32_t)__builtin_amdgcn_mov_dpp(x, 0x55, 0xF, 0xF, true));
  out[2] = bits_f((uint32_t)__builtin_amdgcn_mov_dpp(x, 0xAA, 0xF, 0xF, true));
  out[3] = bits_f((uint32_t)__builtin_amdgcn_mov_dpp(x, 0xFF, 0xF, 0xF, true));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = f_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_to_f(uint32_t h) { return bits_f(h << 16); }

// Two floats -> two OCP e4m3 bytes in the low (hi_word = false) or high half of `old`
// (v_cvt_pk_fp8_f32, round to nearest even).
template <bool hi_word>
__device__ __forceinline__ int cvt_pk_e4m3(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, hi_word);
}
// Byte `sel` of a word of e4m3 codes -> float (v_cvt_f32_fp8).
template <int sel>
__device__ __forceinline__ float e4m3_to_f(int word) {
  return __builtin_amdgcn_cvt_f32_fp8(word, sel);
}

// Four floats as one word of e4m3 codes: hi(y) = the nearest e4m3 values when lo is false,
// the nearest e4m3 values of the residuals y - hi(y) when lo is true (RNE).  `scratch` is
// any dead value: the conversion keeps the other half of its destination, so passing a
// dead register spares the move that would clear it.
__device__ __forceinline__ int e4m3_hilo_word(float y0, float y1, float y2, float y3, bool lo,
                                              int scratch) {
  int hw = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, scratch, false);
  hw = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, hw, true);
  const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, false);
  const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hw, true);
  const float c = lo ? -1.f : 0.f;  // y - hi(y) for lo, y itself (exactly) for hi
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fmaf(c, h01[0], y0), fmaf(c, h01[1], y1), hw, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(fmaf(c, h23[0], y2), fmaf(c, h23[1], y3), w, true);
}

// max(a, b, c) in one v_max3_f32.  fmaxf would first quiet each operand that the compiler
// cannot prove is no signalling NaN (one extra instruction per operand).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// 4x4 byte transpose: in[j] holds bytes (m = 0..3) of token j; out[m] holds byte m of
// tokens 0..3 (byte j of out[m] = byte m of in[j]).
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x06020400u);  // a0b0 a1b0 a0b2 a1b2
  const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030501u);  // a0b1 a1b1 a0b3 a1b3
  const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x06020400u);  // a2b0 a3b0 a2b2 a3b2
  const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030501u);  // a2b1 a3b1 a2b3 a3b3
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[2] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[1] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// Same transpose with per-lane second-stage selectors: (0x05040100, 0x07060302) gives
// tokens in input order 0,1,2,3; (0x01000504, 0x03020706) gives input order 2,3,0,1.
__device__ __forceinline__ void transpose4x4_bytes_sel(const uint32_t in[4], uint32_t out[4],
                                                       uint32_t sel_a, uint32_t sel_b) {
  const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x06020400u);
  const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030501u);
  const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x06020400u);
  const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030501u);
  out[0] = __builtin_amdgcn_perm(t2, t0, sel_a);
  out[2] = __builtin_amdgcn_perm(t2, t0, sel_b);
  out[1] = __builtin_amdgcn_perm(t3, t1, sel_a);
  out[3] = __builtin_amdgcn_perm(t3, t1, sel_b);
}

// Swap a value with the neighbouring lane (lane 2k <-> 2k+1; DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ int swap_adjacent(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);
}

template <typename T>
__device__ __forceinline__ T nt_load(const T* p) {
  return __builtin_nontemporal_load(p);
}

}  // namespace uq

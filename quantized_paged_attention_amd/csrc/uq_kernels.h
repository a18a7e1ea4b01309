// uq_kernels.h -- internal launchers of the libuq kernels (host side, C++ linkage).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uq {

constexpr int kTileGroup = 256;  // tokens per tile-group (partition granule)

struct DecodeArgs {
  const void* q;
  int64_t q_ss, q_sh;          // element strides of the query (sequence, head)
  const uint8_t* cache;
  int64_t blk_stride;          // bytes per physical block = block_size * pos_stride
  int32_t pos_stride;          // bytes per token position = num_kv_heads * slot_bytes
  int32_t slot_bytes;
  const float* k_scale;        // nullable device scalars, or per-token scale tensors
  const float* v_scale;        // [num_blocks, Hk, block_size] (fp8 per-token format)
  const int8_t* rot_signs;     // nullable
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t B, Hk, QG, P, TGPP, max_seq_len, block_size;
  int32_t QL;       // query rows per sequence: unit rows r = j * QG + g, query row b*QL + j
                    // sees tokens t < L_b - QL + 1 + j
  int32_t runs;     // work items per (sequence, kv head)
  int32_t run_len;  // partitions per work item when each partition is one tile-group, else 0
  int32_t head_groups;  // fp8: 1 = a workgroup's waves are consecutive kv heads of one run
  int32_t row_base;     // fp8: first unit row of this launch (without head groups, wide
                        // groups run in passes of 16 rows; set by the launcher)
  int32_t row_splits;   // fp8 head groups: 2 = one launch in which each kv head's 33-64
                        // rows are split over two waves of a workgroup (32 rows each, in
                        // f16 row tiles; 2 kv heads per workgroup); 0 or 1 = one wave per
                        // kv head (up to 32 rows)
  int32_t balanced_items;  // fp8 head groups: > 0 = the partitions of all sequences are
                           // split on the device into this many equal slices per head group
  float softmax_scale;
  uint16_t* part_o;            // bf16 [B, Hk, P, QL*QG, D]
  float* part_m;               // [B, Hk, P, QL*QG]
  float* part_l;
  // Fused flash-combine (fp8 head groups, uq_paged_attention): every work unit of a
  // (sequence, kv head) that does not cover the whole sequence leaves its softmax state
  // in a slot and counts its partitions into counters[b * Hk + h]; the unit that brings
  // the count to the sequence's partition count merges the states and writes the output
  // rows (query dtype) itself, then resets the counter to zero.
  int32_t fused;               // 1: the above; 0: write partials
  void* out;                   // [B*QL, Hq, D] of the query dtype, element strides o_ss, o_sh
  int64_t o_ss, o_sh;
  int32_t* counters;           // [B * Hk * RS], zero between calls (RS = row_splits or 1)
  uint8_t* states;             // kStateBytes per (slot, kv head, row slice, row tile)
  int32_t state_tiles;         // row tiles per state (1 or 2)
};

// One fused state: per lane of the wave, 32 fp32 accumulators (8 x f32x4, lane-major)
// and the (reference, sum) pair of its column.
constexpr int kStateBytes = 8 * 64 * 16 + 2 * 64 * 4;

struct ReduceArgs {
  const uint16_t* part_o;
  const float* part_m;
  const float* part_l;
  const int32_t* seq_lens;
  int32_t B, Hk, QG, D, P, max_seq_len;  // QG: partial rows per (sequence, kv head)
  int32_t QL;       // query rows per sequence (QG a multiple of QL): row r goes to output
                    // row b*QL + r / (QG/QL), head h*(QG/QL) + r % (QG/QL)
  void* out;
  int64_t o_ss, o_sh;
};

struct IndexArgs {
  const uint8_t* q;
  int64_t q_st, q_sh;          // byte strides
  const uint8_t* pages;
  int64_t page_stride;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* seq_lens;
  int32_t num_reqs, QL, H, max_blocks;
  float* scores;
  int64_t s_sh, s_st;
  int32_t cus;                 // compute units of the device (> 0, up to 64 requests: one
                               // wave per live page)
};

// Each returns the hipError_t of its launch.
hipError_t launch_decode_fp8(const DecodeArgs& a, bool q_is_f32, bool tok_scales, hipStream_t stream);
hipError_t launch_decode_fp4(const DecodeArgs& a, bool q_is_f32, bool ue8m0, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, bool out_is_f32, hipStream_t stream);
hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream);

}  // namespace uq

// uq_abi.cpp -- the C ABI of libuq.so (declared in include/uq_paged.h): host-side
// validation, derived launch parameters and kernel launches.  No allocation, no
// synchronisation, no per-call state.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/uq_paged.h"
#include "uq_kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return UQ_OK;
}

int launch_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(UQ_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Compute units of the current device (queried once per device; 256 on MI355X).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

bool valid_block_size(int bs) {
  return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

int slot_content(int fmt, int D) {
  if (fmt == UQ_KV_FP8_E4M3 || fmt == UQ_KV_FP8_E4M3_TOKSCALE) return 2 * D;
  if (fmt == UQ_KV_FP4_E2M1_E4M3S || fmt == UQ_KV_FP4_E2M1_UE8M0S)
    return D % 32 ? -1 : 2 * (D / 2 + D / 32);
  return -1;
}

}  // namespace

extern "C" {

const char* uq_last_error(void) { return g_err; }

size_t uq_decode_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t qg,
                                 int32_t head_dim, int32_t num_partitions) {
  if (num_seqs < 0 || num_kv_heads <= 0 || qg <= 0 || head_dim <= 0 || num_partitions <= 0)
    return 0;
  const size_t rows = (size_t)num_seqs * num_kv_heads * num_partitions * qg;
  return up256(rows * head_dim * 2) + 2 * up256(rows * 4);
}

}  // extern "C"

namespace {

// Work decomposition of a decode launch, from sizes alone (the launches and the workspace
// size of uq_paged_attention share it).
struct Plan {
  int TGPP;            // tile-groups per partition
  int run_len, runs;   // partitions per work item (0: one partition, strided tile-groups)
  int head_groups;     // fp8: workgroups of 4 / row_splits neighbouring kv heads
  int row_splits;      // fp8 head groups: waves per kv head (up to 32 query rows each)
  int balanced_items;  // fp8 head groups: slices per head group (0: runs per sequence)
};

Plan plan_decode(int fmt, int B, int Hk, int P, int max_seq_len, int rows) {
  Plan p{};
  const int ntg = (max_seq_len + uq::kTileGroup - 1) / uq::kTileGroup;
  p.TGPP = ntg == 0 ? 1 : (ntg + P - 1) / P;
  const int pmax = P < ntg ? P : (ntg > 0 ? ntg : 1);
  // Work items: with one tile-group per partition a wave streams a run of consecutive
  // partitions of one (sequence, kv head), so the per-item start-up chain (length ->
  // block table -> first KV loads) is paid once per run and fewer partial rows are
  // written.  Measured on MI355X (B=16 / B=128, ctx up to 16k, 64 partitions): runs of
  // three pay off from 128 partitions per compute unit, runs of two from 16 (shorter
  // grids would leave compute units idle at the end).
  if (p.TGPP == 1) {
    const int64_t work = (int64_t)B * Hk * pmax;
    p.run_len = work >= 128 * 256 ? 3 : (work >= 16 * 256 ? 2 : 1);
    p.runs = (pmax + p.run_len - 1) / p.run_len;
  } else {
    p.run_len = 0;
    p.runs = P;
  }
  if (fmt == UQ_KV_FP8_E4M3 || fmt == UQ_KV_FP8_E4M3_TOKSCALE) {
    // Head groups: with Hk a multiple of 4 a workgroup's 4 waves stream 4 neighbouring kv
    // heads of one (sequence, run of partitions), so they read the neighbouring slots of
    // the same blocks together (a load-only kernel measured 6.2 -> 6.6 TB/s for this
    // order), and each wave writes its own merged partial.  The run length sets how the
    // workgroups pack onto the compute units.  With little work per compute unit, about
    // one workgroup per unit with equal runs; with much, enough runs for two rounds of the
    // three resident workgroups per unit, so that the dispatcher evens out ragged
    // lengths.  Measured on MI355X (fp8, Hk=8, 64 partitions): B=16, L=16k: run 8
    // (256 workgroups) 86 us, runs 4 / 6 / 16: 89 / 102 / 129 us; B=128, L ~ U[4k, 16k]:
    // run 11 472 us, runs 8 / 16 / 22: 482 / 494 / 506 us.
    //   A wave carries up to 32 query rows (two f16 tiles of 16 rows).  Wider groups
    // split their rows over RS = 2 waves of a workgroup (2 kv heads each): one launch
    // reads the KV stream once from HBM, the sibling wave of a head hits the caches, and
    // balanced slices put two workgroups on each compute unit (a wave is latency-bound,
    // so a unit needs four kv heads in flight).  Measured on MI355X (B=128, Hk=8,
    // L ~ U[4k, 16k], fused step): QG=32 454 us with one workgroup per unit, 476 us with
    // two; QG=64 688 us either way.  Before the f16 tiles (e4m3 tiles of 8 rows, 16 rows
    // per wave): QG=32 as passes of 16 rows 915 us, 2 row slices with two workgroups per
    // unit 658 us; QG=64 1836 / 1108 us (4 row slices).
    const int RS = rows <= 32 ? 1 : 2;
    const int HPW = 4 / RS;
    if (Hk % HPW == 0) {
      p.head_groups = 1;
      p.row_splits = RS;
      if (p.TGPP == 1 && B > 0) {
        const int64_t units = (int64_t)B * (Hk / HPW);  // workgroups per run
        const int64_t cus = device_cus();
        int64_t G;  // runs per (sequence, head group)
        if (units * pmax <= 16 * cus)
          G = (cus + units - 1) / units;
        else
          G = (6 * cus + units - 1) / units;
        G = G < 1 ? 1 : (G > pmax ? pmax : G);
        p.run_len = (int)((pmax + G - 1) / G);
        p.runs = (pmax + p.run_len - 1) / p.run_len;
        // With much work, balanced slices instead: one workgroup per compute unit, each
        // taking an equal share of all sequences' partitions (split on the device from
        // the lengths, up to 16 per lane: B <= 1024), so ragged lengths leave no tail.
        // Measured on MI355X (B=128, L ~ U[4k, 16k]): decode 469 -> 409 us; two or three
        // workgroups per unit 439 / 453 us.  With little work the runs above already fill
        // one round (B=16, L=16k: 88 us either way).
        if (units * pmax > 16 * cus && B <= 1024) {
          const int64_t per_hg = (RS > 1 ? 2 : 1) * cus / (Hk / HPW);
          p.balanced_items = (int)(per_hg > 0 ? per_hg : 1);
        }
      }
    }
  } else if (p.TGPP == 1) {
    // FP4: one workgroup streams a run of R partitions (one query rotation, one merged
    // partial).  Two workgroups fit a compute unit, and the time goes as (rounds of
    // resident workgroups) x (R + about one partition of fixed cost per workgroup:
    // rotation, start-up, merge), so R in [1, 8] minimises ceil(groups / slots) * (R + 1)
    // (ties: the shorter run).  Measured on MI355X (B=4, Hk=2, ctx 75000, 512 partitions,
    // 512 slots, 20 launches back to back): R = 5 (472 groups, one round) 38.6 us;
    // R = 3, 4, 6, 8: 51.7, 48.9, 42.3, 50.9 us.
    const int64_t slots = 2LL * device_cus();
    int best_r = 1;
    int64_t best_cost = -1;
    for (int r = 1; r <= 8; ++r) {
      const int64_t groups = (int64_t)B * Hk * ((pmax + r - 1) / r);
      const int64_t cost = (groups + slots - 1) / slots * (r + 1);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best_r = r;
      }
    }
    p.run_len = best_r;
    p.runs = (pmax + p.run_len - 1) / p.run_len;
  }
  return p;
}

// Workspace of uq_paged_attention: a fixed region of arrival counters (the fp8 fused
// step: [B, Hk, row slices]), then either the fused states (fp8 head groups: one slot per
// work unit of a sequence, kStateBytes per kv head, row slice and row tile) or the three
// decode partial buffers.
// The counter region has the same size for every call, and nothing else is ever written
// there, so the zeros that each completed call leaves in it hold for a later call of any
// sizes (a region that grew with the sizes would take in the bodies of earlier, smaller
// calls).  A call that needs more counters than the region holds runs the two-launch
// decode + reduce instead.
constexpr size_t kCounterBytes = (size_t)256 << 10;

struct AttnLayout {
  bool fused;
  int tiles;              // row tiles per fused state
  int64_t slots;          // fused state slots
  size_t counter_bytes, body_bytes;
};

AttnLayout attn_layout(int fmt, int B, int Hk, int QL, int QG, int D, int P, int max_seq_len) {
  AttnLayout l{};
  const int64_t rows64 = (int64_t)QL * QG;
  const int rows = rows64 > 1024 ? 1024 : (int)rows64;
  const Plan p = plan_decode(fmt, B, Hk, P, max_seq_len, rows);
  const int RS = p.row_splits > 1 ? p.row_splits : 1;
  l.counter_bytes = kCounterBytes;
  l.fused = (fmt == UQ_KV_FP8_E4M3 || fmt == UQ_KV_FP8_E4M3_TOKSCALE) && p.head_groups &&
            (size_t)B * Hk * RS * 4 <= kCounterBytes;
  if (l.fused) {
    l.tiles = rows <= 16 ? 1 : 2;  // e4m3 tiles of 8 rows up to 8, f16 tiles of 16 above
    // balanced slices: unit (b, slice s) uses slot s + b; runs: unit (b, run g) slot
    // b * runs + g
    l.slots = p.balanced_items > 0 ? (int64_t)p.balanced_items + B - 1 : (int64_t)B * p.runs;
    if (l.slots < 1) l.slots = 1;
    l.body_bytes = up256((size_t)l.slots * Hk * RS * l.tiles * uq::kStateBytes);
  } else {
    l.body_bytes = uq_decode_workspace_bytes(B, Hk, rows, D, P);
  }
  return l;
}

}  // namespace

extern "C" {

size_t uq_attention_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t query_len,
                                    int32_t qg, int32_t head_dim, int32_t num_partitions,
                                    int32_t max_seq_len, int kv_format) {
  if (num_seqs < 0 || num_kv_heads <= 0 || query_len < 1 || qg <= 0 || head_dim <= 0 ||
      num_partitions <= 0 || max_seq_len < 0 || slot_content(kv_format, head_dim) < 0)
    return 0;
  const AttnLayout l = attn_layout(kv_format, num_seqs, num_kv_heads, query_len, qg, head_dim,
                                   num_partitions, max_seq_len);
  return l.counter_bytes + l.body_bytes;
}

}  // extern "C"

namespace {

// Validation and launch of the decode kernels.  Without `fused` the partial buffers are
// the outputs; with it the fp8 head-group kernels finish the flash-combine themselves
// and write `fused->out` (the caller has checked that the layout is fused).
struct FusedTarget {
  void* out;
  int64_t o_ss, o_sh;
  int32_t* counters;
  uint8_t* states;
  int tiles;
};

int decode_impl(const void* query, int q_dtype, int64_t q_stride_seq, int64_t q_stride_head,
                const uint8_t* kv_cache, int64_t num_blocks, int32_t block_size,
                int32_t num_kv_heads, int32_t slot_bytes, int kv_format, const float* k_scale,
                const float* v_scale, const int8_t* rot_signs, const int32_t* block_table,
                int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                int32_t query_len, int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                float softmax_scale, int32_t num_partitions, void* part_out, float* part_max,
                float* part_sum, const FusedTarget* fused, void* stream) {
  if (num_seqs < 0) return fail(UQ_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (query_len < 1) return fail(UQ_ERR_INVALID_ARG, "query_len must be >= 1 (got %d)", query_len);
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(UQ_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  const int QG = num_q_heads / num_kv_heads;
  if (QG > 64) return fail(UQ_ERR_INVALID_ARG, "query group %d exceeds 64", QG);
  if (q_dtype != UQ_F32 && q_dtype != UQ_BF16)
    return fail(UQ_ERR_INVALID_ARG, "q_dtype must be UQ_F32 or UQ_BF16 (got %d)", q_dtype);
  if (q_stride_seq <= 0 || q_stride_head <= 0)
    return fail(UQ_ERR_INVALID_ARG, "query strides must be positive");
  if (!valid_block_size(block_size))
    return fail(UQ_ERR_INVALID_ARG, "block_size must be 16, 32, 64, 128 or 256 (got %d)", block_size);
  if (num_blocks <= 0) return fail(UQ_ERR_INVALID_ARG, "num_blocks must be positive");
  const int content = slot_content(kv_format, head_dim);
  if (content < 0) return fail(UQ_ERR_INVALID_ARG, "unknown kv_format %d or head_dim %d", kv_format, head_dim);
  if (slot_bytes < content || slot_bytes % 4 != 0)
    return fail(UQ_ERR_INVALID_ARG, "slot_bytes %d must be >= %d and a multiple of 4", slot_bytes, content);
  if (num_partitions < 1) return fail(UQ_ERR_INVALID_ARG, "num_partitions must be >= 1");
  if (max_seq_len < 0) return fail(UQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (bt_stride <= 0 || (int64_t)bt_stride * block_size < max_seq_len)
    return fail(UQ_ERR_INVALID_ARG, "bt_stride %d cannot hold max_seq_len %d at block size %d",
                bt_stride, max_seq_len, block_size);
  if (!std::isfinite(softmax_scale)) return fail(UQ_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (num_seqs > 0 && (!query || !kv_cache || !block_table || !seq_lens))
    return fail(UQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (!fused && num_seqs > 0 && (!part_out || !part_max || !part_sum))
    return fail(UQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(query) | reinterpret_cast<uintptr_t>(part_out)) & 15)
    return fail(UQ_ERR_INVALID_ARG, "query and part_out must be 16-byte aligned");
  const int esz = q_dtype == UQ_F32 ? 4 : 2;
  if (((q_stride_seq * esz) | (q_stride_head * esz)) % 16)
    return fail(UQ_ERR_INVALID_ARG, "query strides must be multiples of 16 bytes");
  if (reinterpret_cast<uintptr_t>(kv_cache) & 15)
    return fail(UQ_ERR_INVALID_ARG, "kv_cache must be 16-byte aligned");

  const int64_t rows64 = (int64_t)query_len * QG;
  const Plan plan = plan_decode(kv_format, num_seqs, num_kv_heads, num_partitions, max_seq_len,
                                rows64 > 1024 ? 1024 : (int)rows64);
  uq::DecodeArgs a{};
  a.q = query;
  a.q_ss = q_stride_seq;
  a.q_sh = q_stride_head;
  a.cache = kv_cache;
  a.slot_bytes = slot_bytes;
  a.pos_stride = num_kv_heads * slot_bytes;
  a.blk_stride = (int64_t)block_size * a.pos_stride;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.rot_signs = rot_signs;
  a.bt = block_table;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.B = num_seqs;
  a.Hk = num_kv_heads;
  a.QG = QG;
  a.QL = query_len;
  a.P = num_partitions;
  a.TGPP = plan.TGPP;
  a.max_seq_len = max_seq_len;
  a.block_size = block_size;
  a.run_len = plan.run_len;
  a.runs = plan.runs;
  a.head_groups = plan.head_groups;
  a.row_splits = plan.row_splits;
  a.balanced_items = plan.balanced_items;
  a.softmax_scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  a.part_o = static_cast<uint16_t*>(part_out);
  a.part_m = part_max;
  a.part_l = part_sum;
  if (fused) {
    a.fused = 1;
    a.out = fused->out;
    a.o_ss = fused->o_ss;
    a.o_sh = fused->o_sh;
    a.counters = fused->counters;
    a.states = fused->states;
    a.state_tiles = fused->tiles;
  }
  if ((int64_t)a.pos_stride * block_size > (int64_t)1 << 31)
    return fail(UQ_ERR_UNSUPPORTED, "a physical block larger than 2 GiB is not supported");

  if (kv_format == UQ_KV_FP8_E4M3 || kv_format == UQ_KV_FP8_E4M3_TOKSCALE) {
    const bool tok = kv_format == UQ_KV_FP8_E4M3_TOKSCALE;
    if (tok && num_seqs > 0 && (!k_scale || !v_scale))
      return fail(UQ_ERR_INVALID_ARG, "per-token scales need both k_scale and v_scale tensors");
    if ((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 3)
      return fail(UQ_ERR_INVALID_ARG, "k_scale and v_scale must be 4-byte aligned");
    if (head_dim != 128) return fail(UQ_ERR_UNSUPPORTED, "fp8 cache supports head_dim 128 only");
    if (query_len * QG > 64)
      return fail(UQ_ERR_UNSUPPORTED, "fp8 cache supports query_len x query group up to 64 rows (got %d x %d)",
                  query_len, QG);
    if (rot_signs) return fail(UQ_ERR_UNSUPPORTED, "query rotation is supported with fp4 caches only");
    if (slot_bytes % 16) return fail(UQ_ERR_UNSUPPORTED, "fp8 cache needs slot_bytes a multiple of 16");
    if (num_seqs == 0) return ok();
    return launch_status(uq::launch_decode_fp8(a, q_dtype == UQ_F32, tok, static_cast<hipStream_t>(stream)),
                         "decode_fp8");
  }
  if (kv_format == UQ_KV_FP4_E2M1_E4M3S || kv_format == UQ_KV_FP4_E2M1_UE8M0S) {
    if (head_dim != 256) return fail(UQ_ERR_UNSUPPORTED, "fp4 cache supports head_dim 256 only");
    if (k_scale || v_scale) return fail(UQ_ERR_INVALID_ARG, "per-tensor scales apply to fp8 caches only");
    if (reinterpret_cast<uintptr_t>(rot_signs) & 15)
      return fail(UQ_ERR_INVALID_ARG, "rot_signs must be 16-byte aligned");
    if (slot_bytes % 16) return fail(UQ_ERR_UNSUPPORTED, "fp4 cache needs slot_bytes a multiple of 16");
    if (query_len * QG > 16)
      return fail(UQ_ERR_UNSUPPORTED, "fp4 cache supports query_len x query group up to 16 rows (got %d x %d)",
                  query_len, QG);
    if (fused) return fail(UQ_ERR_UNSUPPORTED, "the fused flash-combine covers fp8 head groups only");
    if (num_seqs == 0) return ok();
    return launch_status(uq::launch_decode_fp4(a, q_dtype == UQ_F32, kv_format == UQ_KV_FP4_E2M1_UE8M0S,
                                               static_cast<hipStream_t>(stream)),
                         "decode_fp4");
  }
  return fail(UQ_ERR_UNSUPPORTED, "kv_format %d is not implemented", kv_format);
}

}  // namespace

extern "C" {

int uq_paged_decode_mtp(const void* query, int q_dtype, int64_t q_stride_seq,
                        int64_t q_stride_head, const uint8_t* kv_cache, int64_t num_blocks,
                        int32_t block_size, int32_t num_kv_heads, int32_t slot_bytes,
                        int kv_format, const float* k_scale, const float* v_scale,
                        const int8_t* rot_signs, const int32_t* block_table, int32_t bt_stride,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t query_len,
                        int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                        float softmax_scale, int32_t num_partitions, void* part_out,
                        float* part_max, float* part_sum, void* stream) {
  return decode_impl(query, q_dtype, q_stride_seq, q_stride_head, kv_cache, num_blocks,
                     block_size, num_kv_heads, slot_bytes, kv_format, k_scale, v_scale, rot_signs,
                     block_table, bt_stride, seq_lens, num_seqs, query_len, num_q_heads, head_dim,
                     max_seq_len, softmax_scale, num_partitions, part_out, part_max, part_sum,
                     nullptr, stream);
}

int uq_paged_decode(const void* query, int q_dtype, int64_t q_stride_seq, int64_t q_stride_head,
                    const uint8_t* kv_cache, int64_t num_blocks, int32_t block_size,
                    int32_t num_kv_heads, int32_t slot_bytes, int kv_format,
                    const float* k_scale, const float* v_scale, const int8_t* rot_signs,
                    const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                    int32_t max_seq_len, float softmax_scale, int32_t num_partitions,
                    void* part_out, float* part_max, float* part_sum, void* stream) {
  return uq_paged_decode_mtp(query, q_dtype, q_stride_seq, q_stride_head, kv_cache, num_blocks,
                             block_size, num_kv_heads, slot_bytes, kv_format, k_scale, v_scale,
                             rot_signs, block_table, bt_stride, seq_lens, num_seqs, 1, num_q_heads,
                             head_dim, max_seq_len, softmax_scale, num_partitions, part_out,
                             part_max, part_sum, stream);
}

int uq_paged_reduce_mtp(const void* part_out, const float* part_max, const float* part_sum,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                        int32_t query_len, int32_t qg, int32_t head_dim, int32_t num_partitions,
                        int32_t max_seq_len, void* out, int out_dtype, int64_t o_stride_seq,
                        int64_t o_stride_head, void* stream) {
  if (query_len < 1) return fail(UQ_ERR_INVALID_ARG, "query_len must be >= 1 (got %d)", query_len);
  if (num_seqs < 0 || num_kv_heads <= 0 || qg < 1 || query_len * qg > 64)
    return fail(UQ_ERR_INVALID_ARG, "bad sizes: num_seqs %d, num_kv_heads %d, query_len %d x qg %d",
                num_seqs, num_kv_heads, query_len, qg);
  if (head_dim != 128 && head_dim != 256)
    return fail(UQ_ERR_UNSUPPORTED, "reduce supports head_dim 128 and 256 (got %d)", head_dim);
  if (num_partitions < 1) return fail(UQ_ERR_INVALID_ARG, "num_partitions must be >= 1");
  if (max_seq_len < 0) return fail(UQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (out_dtype != UQ_F32 && out_dtype != UQ_BF16)
    return fail(UQ_ERR_INVALID_ARG, "out_dtype must be UQ_F32 or UQ_BF16 (got %d)", out_dtype);
  if (o_stride_seq <= 0 || o_stride_head <= 0)
    return fail(UQ_ERR_INVALID_ARG, "output strides must be positive");
  if (num_seqs > 0 && (!part_out || !part_max || !part_sum || !seq_lens || !out))
    return fail(UQ_ERR_INVALID_ARG, "a required pointer is NULL");
  const int esz = out_dtype == UQ_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(part_out)) & 15 ||
      ((o_stride_seq * esz) | (o_stride_head * esz)) % 16)
    return fail(UQ_ERR_INVALID_ARG, "out, part_out and the output strides must be 16-byte aligned");
  if (num_seqs == 0) return ok();
  uq::ReduceArgs a{};
  a.part_o = static_cast<const uint16_t*>(part_out);
  a.part_m = part_max;
  a.part_l = part_sum;
  a.seq_lens = seq_lens;
  a.B = num_seqs;
  a.Hk = num_kv_heads;
  a.QG = query_len * qg;  // partial rows per (sequence, kv head)
  a.QL = query_len;
  a.D = head_dim;
  a.P = num_partitions;
  a.max_seq_len = max_seq_len;
  a.out = out;
  a.o_ss = o_stride_seq;
  a.o_sh = o_stride_head;
  return launch_status(uq::launch_reduce(a, out_dtype == UQ_F32, static_cast<hipStream_t>(stream)),
                       "reduce");
}

int uq_paged_reduce(const void* part_out, const float* part_max, const float* part_sum,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads, int32_t qg,
                    int32_t head_dim, int32_t num_partitions, int32_t max_seq_len, void* out,
                    int out_dtype, int64_t o_stride_seq, int64_t o_stride_head, void* stream) {
  return uq_paged_reduce_mtp(part_out, part_max, part_sum, seq_lens, num_seqs, num_kv_heads, 1, qg,
                             head_dim, num_partitions, max_seq_len, out, out_dtype, o_stride_seq,
                             o_stride_head, stream);
}

int uq_paged_attention(const void* query, int q_dtype, int64_t q_stride_seq,
                       int64_t q_stride_head, const uint8_t* kv_cache, int64_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t slot_bytes,
                       int kv_format, const float* k_scale, const float* v_scale,
                       const int8_t* rot_signs, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t query_len,
                       int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                       float softmax_scale, int32_t num_partitions, void* workspace,
                       size_t workspace_bytes, void* out, int64_t o_stride_seq,
                       int64_t o_stride_head, void* stream) {
  if (num_seqs < 0) return fail(UQ_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (query_len < 1) return fail(UQ_ERR_INVALID_ARG, "query_len must be >= 1 (got %d)", query_len);
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(UQ_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  if (q_dtype != UQ_F32 && q_dtype != UQ_BF16)
    return fail(UQ_ERR_INVALID_ARG, "q_dtype must be UQ_F32 or UQ_BF16 (got %d)", q_dtype);
  if (num_partitions < 1) return fail(UQ_ERR_INVALID_ARG, "num_partitions must be >= 1");
  if (max_seq_len < 0) return fail(UQ_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (slot_content(kv_format, head_dim) < 0)
    return fail(UQ_ERR_INVALID_ARG, "unknown kv_format %d or head_dim %d", kv_format, head_dim);
  if (o_stride_seq <= 0 || o_stride_head <= 0)
    return fail(UQ_ERR_INVALID_ARG, "output strides must be positive");
  const int esz = q_dtype == UQ_F32 ? 4 : 2;
  if (num_seqs > 0 && (!out || !workspace))
    return fail(UQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(out) & 15) || ((o_stride_seq * esz) | (o_stride_head * esz)) % 16)
    return fail(UQ_ERR_INVALID_ARG, "out and the output strides must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(UQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const int QG = num_q_heads / num_kv_heads;
  const AttnLayout l = attn_layout(kv_format, num_seqs, num_kv_heads, query_len, QG, head_dim,
                                   num_partitions, max_seq_len);
  if (workspace_bytes < l.counter_bytes + l.body_bytes)
    return fail(UQ_ERR_INVALID_ARG, "workspace of %zu bytes is below the %zu this call needs",
                workspace_bytes, l.counter_bytes + l.body_bytes);
  if (num_seqs == 0) return ok();
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  if (l.fused) {
    FusedTarget ft{out, o_stride_seq, o_stride_head, reinterpret_cast<int32_t*>(ws),
                   ws + l.counter_bytes, l.tiles};
    return decode_impl(query, q_dtype, q_stride_seq, q_stride_head, kv_cache, num_blocks,
                       block_size, num_kv_heads, slot_bytes, kv_format, k_scale, v_scale,
                       rot_signs, block_table, bt_stride, seq_lens, num_seqs, query_len,
                       num_q_heads, head_dim, max_seq_len, softmax_scale, num_partitions,
                       nullptr, nullptr, nullptr, &ft, stream);
  }
  // decode into partials carved from the workspace, then the flash-combine launch
  const size_t rows = (size_t)num_seqs * num_kv_heads * num_partitions * query_len * QG;
  uint8_t* po = ws + l.counter_bytes;
  float* pm = reinterpret_cast<float*>(po + up256(rows * head_dim * 2));
  float* pl = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(pm) + up256(rows * 4));
  int st = decode_impl(query, q_dtype, q_stride_seq, q_stride_head, kv_cache, num_blocks,
                       block_size, num_kv_heads, slot_bytes, kv_format, k_scale, v_scale,
                       rot_signs, block_table, bt_stride, seq_lens, num_seqs, query_len,
                       num_q_heads, head_dim, max_seq_len, softmax_scale, num_partitions, po, pm,
                       pl, nullptr, stream);
  if (st != UQ_OK) return st;
  return uq_paged_reduce_mtp(po, pm, pl, seq_lens, num_seqs, num_kv_heads, query_len, QG,
                             head_dim, num_partitions, max_seq_len, out, q_dtype, o_stride_seq,
                             o_stride_head, stream);
}

int uq_index_score(const uint8_t* q, int64_t q_stride_tok, int64_t q_stride_head,
                   const uint8_t* k_pages, int64_t page_stride, int64_t num_pages,
                   const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                   int32_t num_reqs, int32_t query_len, int32_t heads, int32_t head_dim,
                   int32_t init_blocks, int32_t local_blocks, float* scores,
                   int64_t s_stride_head, int64_t s_stride_row, int32_t max_blocks,
                   void* stream) {
  if (num_reqs < 0) return fail(UQ_ERR_INVALID_ARG, "num_reqs must be >= 0");
  if (heads != 1 && heads != 2 && heads != 4)
    return fail(UQ_ERR_INVALID_ARG, "heads must be 1, 2 or 4 (got %d)", heads);
  if (query_len < 1 || heads * query_len > 32)
    return fail(UQ_ERR_INVALID_ARG, "heads * query_len must be in [1, 32] (got %d x %d)", heads,
                query_len);
  if (head_dim != 128) return fail(UQ_ERR_UNSUPPORTED, "index scorer supports head_dim 128 only");
  if (init_blocks != 0 || local_blocks != 0)
    return fail(UQ_ERR_UNSUPPORTED, "sentinel init/local blocks are not supported");
  if (q_stride_tok <= 0 || q_stride_head <= 0 || q_stride_tok % 16 || q_stride_head % 16)
    return fail(UQ_ERR_INVALID_ARG, "q strides must be positive multiples of 16 bytes");
  // one request's query rows are addressed with 32-bit offsets
  if ((int64_t)(query_len - 1) * q_stride_tok + (int64_t)(heads - 1) * q_stride_head + head_dim >
      0x7FFFFFFFLL)
    return fail(UQ_ERR_UNSUPPORTED, "a request's query rows span more than 2^31 - 1 bytes");
  const int64_t content = 128LL * (head_dim / 2 + head_dim / 16);
  if (page_stride < content || page_stride % 16)
    return fail(UQ_ERR_INVALID_ARG, "page_stride %lld must be >= %lld and a multiple of 16",
                (long long)page_stride, (long long)content);
  if (num_pages <= 0 || bt_stride <= 0 || max_blocks <= 0)
    return fail(UQ_ERR_INVALID_ARG, "num_pages, bt_stride and max_blocks must be positive");
  if (s_stride_head <= 0 || s_stride_row <= 0)
    return fail(UQ_ERR_INVALID_ARG, "score strides must be positive");
  // rows of max_blocks cells must not overlap, nor the [rows, max_blocks] planes of heads
  if (s_stride_row < max_blocks)
    return fail(UQ_ERR_INVALID_ARG, "s_stride_row %lld is below max_blocks %d",
                (long long)s_stride_row, max_blocks);
  if (heads > 1 && num_reqs > 0 &&
      s_stride_head < ((int64_t)num_reqs * query_len - 1) * s_stride_row + max_blocks)
    return fail(UQ_ERR_INVALID_ARG, "s_stride_head %lld makes the heads' score planes overlap",
                (long long)s_stride_head);
  if (num_reqs > 0 && (!q || !k_pages || !block_table || !seq_lens || !scores))
    return fail(UQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_pages)) & 15)
    return fail(UQ_ERR_INVALID_ARG, "q and k_pages must be 16-byte aligned");
  if (num_reqs == 0) return ok();
  uq::IndexArgs a{};
  a.q = q;
  a.q_st = q_stride_tok;
  a.q_sh = q_stride_head;
  a.pages = k_pages;
  a.page_stride = page_stride;
  a.bt = block_table;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.num_reqs = num_reqs;
  a.QL = query_len;
  a.H = heads;
  a.max_blocks = max_blocks < bt_stride ? max_blocks : bt_stride;
  a.scores = scores;
  a.s_sh = s_stride_head;
  a.s_st = s_stride_row;
  a.cus = device_cus();  // sizes the one-wave-per-live-page grid
  return launch_status(uq::launch_index_score(a, static_cast<hipStream_t>(stream)), "index_score");
}

}  // extern "C"

// ---- uq_paged_attention_noalloc: the same step with its workspace in a file-scope device
//      array (one copy per GPU, held until the process ends), for callers that cannot
//      allocate.  The host name `scratch` is a stand-in, not a device address: the address
//      of each GPU's copy comes from hipGetSymbolAddress, once per device, with that device
//      current.  The counter region at its start (the same 256 KiB for every call, written
//      by nothing else) is zero from module load and every completed call leaves it zero
//      again; the rest is written before it is read.
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch`, or NULL (the last error set) on failure
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    fail(UQ_ERR_LAUNCH, "no current HIP device (or device index >= %d)", kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(UQ_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int uq_paged_attention_noalloc(const void* query, int q_dtype, int64_t q_stride_seq,
                               int64_t q_stride_head, const uint8_t* kv_cache,
                               int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                               int32_t slot_bytes, int kv_format, const float* k_scale,
                               const float* v_scale, const int8_t* rot_signs,
                               const int32_t* block_table, int32_t bt_stride,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t query_len,
                               int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                               float softmax_scale, int32_t num_partitions, void* out,
                               int64_t o_stride_seq, int64_t o_stride_head, void* stream) {
  if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(UQ_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, num_kv_heads);
  const size_t need = uq_attention_workspace_bytes(num_seqs, num_kv_heads, query_len,
                                                   num_q_heads / num_kv_heads, head_dim,
                                                   num_partitions, max_seq_len, kv_format);
  if (need == 0)
    return fail(UQ_ERR_INVALID_ARG, "invalid sizes (num_seqs %d, query_len %d, head_dim %d, "
                "num_partitions %d, max_seq_len %d, kv_format %d)", num_seqs, query_len,
                head_dim, num_partitions, max_seq_len, kv_format);
  if (need > kScratchBytes)
    return fail(UQ_ERR_INVALID_ARG, "this call needs %zu bytes of workspace, more than the %zu "
                "of the no-allocation scratch; use uq_paged_attention with a workspace",
                need, kScratchBytes);
  if (num_seqs == 0)
    return uq_paged_attention(query, q_dtype, q_stride_seq, q_stride_head, kv_cache, num_blocks,
                              block_size, num_kv_heads, slot_bytes, kv_format, k_scale, v_scale,
                              rot_signs, block_table, bt_stride, seq_lens, num_seqs, query_len,
                              num_q_heads, head_dim, max_seq_len, softmax_scale, num_partitions,
                              nullptr, 0, out, o_stride_seq, o_stride_head, stream);
  void* ws = scratch_of_current_device();
  if (!ws) return UQ_ERR_LAUNCH;
  return uq_paged_attention(query, q_dtype, q_stride_seq, q_stride_head, kv_cache, num_blocks,
                            block_size, num_kv_heads, slot_bytes, kv_format, k_scale, v_scale,
                            rot_signs, block_table, bt_stride, seq_lens, num_seqs, query_len,
                            num_q_heads, head_dim, max_seq_len, softmax_scale, num_partitions, ws,
                            kScratchBytes, out, o_stride_seq, o_stride_head, stream);
}

}  // extern "C"


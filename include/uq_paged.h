/*
 * uq_paged.h -- C ABI of libuq.so: quantized paged-attention decode and the nvfp4 index
 * scorer for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless noted.
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is enqueued on it;
 *     nothing synchronises the host, nothing allocates device memory, and no per-call
 *     state is kept, so calls may be captured in a HIP graph.
 *   - Arguments are validated on the host before anything is launched.  A rejected call
 *     returns a non-zero uq_status, launches nothing and writes nothing; uq_last_error()
 *     then describes the problem.  Contents of device buffers cannot be checked on the
 *     host: the "device preconditions" listed per entry point are the caller's duty.
 *   - Sizes are element counts unless the name says bytes.
 *
 * Sources (the operations are defined on these pages):
 *   [P1] vLLM PR 59857 API page "ultraquant_decode_hd256": FP4 D=256 GQA decode over an
 *        AoS slot cache, strided partition -> 256-token tile-group map, fused
 *        Walsh-Hadamard query rotation (STEP B'), online softmax (STEP F), partition
 *        epilogue (STEP G).
 *   [P2] vLLM PR 59747 API page "nvfp4_index_decode/kernel": compile_score_decode, the
 *        per-page max of q.k over nvfp4 K pages with a causal limit for trailing rows.
 *   [P3] GitHub ROCm/FlyDSL PR #825 "pa_decode_tile": per-tensor fp8 paged decode,
 *        cross-workgroup partition split + flash-combine reduce, k/v scales as 1-element
 *        device tensors, explicit Q strides, caller-preallocated partials.
 */
#ifndef UQ_PAGED_H
#define UQ_PAGED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
enum {
  UQ_OK = 0,
  UQ_ERR_INVALID_ARG = 1,  /* a pointer, size, stride or dtype is not acceptable        */
  UQ_ERR_UNSUPPORTED = 2,  /* well-formed, but outside what the kernels implement        */
  UQ_ERR_LAUNCH = 3        /* the HIP runtime reported an error at launch                 */
};

/* Floating-point element types of query / output tensors. */
enum { UQ_F32 = 0, UQ_BF16 = 1 };

/* KV cache formats: one AoS slot of `slot_bytes` per (token, kv head).
 *   UQ_KV_FP8_E4M3        K codes [0, D), V codes [D, 2D): OCP e4m3fn with one per-tensor
 *                         scale each ([P3] per-tensor fp8 K/V).  Supported for D = 128.
 *   UQ_KV_FP4_E2M1_E4M3S  K e2m1 codes [0, D/2), K scales [D/2, D/2+D/32), V codes
 *                         [D/2+D/32, D+D/32), V scales [D+D/32, D+D/16): one e4m3 scale
 *                         per 32 dims; element 2i is the low nibble of byte i ([P1] slot
 *                         layout: 0/128/136/264, 272 bytes at D=256).  Supported for
 *                         D = 256.
 *   UQ_KV_FP4_E2M1_UE8M0S same slot with UE8M0 scales 2^(byte-127), byte 0 = 0.0 ([P1]
 *                         STEP F scale words).  Supported for D = 256.
 *   UQ_KV_FP8_E4M3_TOKSCALE  the UQ_KV_FP8_E4M3 slot with one f32 K scale and one f32 V
 *                         scale per (token, kv head) ([P3] per_token_kv mode) held in two
 *                         tensors [num_blocks, num_kv_heads, block_size] (physical block,
 *                         head, position in the block) passed as k_scale / v_scale.
 *                         Supported for D = 128. */
enum { UQ_KV_FP8_E4M3 = 0, UQ_KV_FP4_E2M1_E4M3S = 1, UQ_KV_FP4_E2M1_UE8M0S = 2,
       UQ_KV_FP8_E4M3_TOKSCALE = 3 };

/* uq_paged_decode -- one decode step of paged attention, split over context partitions.
 *
 * Computes, for every sequence b, kv head h, query row g of the GQA group
 * (query head h*QG + g, QG = num_q_heads / num_kv_heads) and partition p, the softmax
 * statistics of the tokens that partition owns ([P1] builder comments and STEP F trip
 * count: partition p owns the 256-token tile-groups p, p+P, p+2P, ...):
 *   s_t  = softmax_scale * k_scale * (q' . k_t),   t < L_b, t in partition p
 *   m    = max_t s_t,   l = sum_t exp(s_t - m),
 *   o    = v_scale * sum_t exp(s_t - m) v_t / l        (rounded to bf16)
 * q' = q, or with rot_signs q' = (q * s) H / sqrt(D), H the Sylvester Hadamard matrix
 * ([P1] STEP B').  k, v are the decoded cache values (e4m3, or e2m1 x group scale).
 *
 *   query         [num_seqs, num_q_heads, head_dim] of q_dtype (UQ_F32 or UQ_BF16),
 *                 element strides q_stride_seq / q_stride_head (> 0; the head dim is
 *                 contiguous).  Q may be a slice of a fused QKV projection ([P1] Q
 *                 strides comment).
 *   kv_cache      [num_blocks, block_size, num_kv_heads, slot_bytes] uint8.  block_size in
 *                 {16, 32, 64, 128, 256}; slot_bytes >= slot content and a multiple of 4.
 *   k_scale,      device float[1] per-tensor scales (UQ_KV_FP8_E4M3), or NULL for 1.0
 *   v_scale       ([P3] scales as 1-element device tensors).  Must be NULL for fp4.
 *                 With UQ_KV_FP8_E4M3_TOKSCALE both are required: device float
 *                 [num_blocks, num_kv_heads, block_size], 4-byte aligned; token t of
 *                 sequence b in head h then decodes as k_t = e4m3(K codes) * k_scale[blk,
 *                 h, t mod block_size], v_t likewise with v_scale (blk = its physical
 *                 block), and s_t = softmax_scale * (q' . k_t).  Scales of visible
 *                 tokens must be finite; those of other slots are never used.
 *   rot_signs     device int8[head_dim] of +-1 for the query rotation, or NULL.
 *                 fp4 formats only; 16-byte aligned.
 *   block_table   [num_seqs, bt_stride] int32 physical block ids.
 *   seq_lens      [num_seqs] int32 context lengths.
 *   max_seq_len   host-side upper bound of seq_lens (>= 0); fixes the tile-groups per
 *                 partition as ceil(ceil(max_seq_len / 256) / num_partitions), so no token
 *                 is ever dropped.
 *   softmax_scale <= 0 selects 1/sqrt(head_dim) ([P1] default scale).
 *   num_partitions P >= 1.
 *   part_out      bf16 [num_seqs, num_kv_heads, P, QG, head_dim]      (workspace, output)
 *   part_max      f32  [num_seqs, num_kv_heads, P, QG]  natural-log-domain maxima m
 *   part_sum      f32  [num_seqs, num_kv_heads, P, QG]  sums l
 * Only partitions that own at least one token (p < ceil(L_b / 256)) are written; the
 * others keep their contents and are never read by uq_paged_reduce.  The partials are a
 * flash-combine workspace: the decode may merge the statistics of a set of consecutive
 * partitions into the first of them (m, l, o of their union) and write the others of the
 * set as empty (m = -inf, l = 0, o rows left unwritten).  Combining all written states
 * with uq_paged_reduce gives the attention output either way.  The kernels merge the
 * run of consecutive partitions streamed for one kv head by one wave (fp8 with head
 * groups: num_kv_heads a multiple of 4, or of 2 for groups of 33-64 rows) or by one
 * workgroup (otherwise); the run length is
 * chosen by the launcher from the problem size and the device's compute units.
 * With num_partitions = 1 part_* hold exactly the statistics above.
 * Supported: (UQ_KV_FP8_E4M3 or UQ_KV_FP8_E4M3_TOKSCALE, D = 128, QG <= 64) and
 * (UQ_KV_FP4_E2M1_E4M3S or UQ_KV_FP4_E2M1_UE8M0S, D = 256, QG <= 16); anything else
 * returns UQ_ERR_UNSUPPORTED ([P3] wide GQA: groups above 16 rows).  The fp8 kernels
 * read the cache once per kv head for all its query rows with head groups (up to 32
 * rows per wave, 33-64 rows on two waves of a workgroup); without head groups a group
 * wider than 16 rows runs one pass per 16 rows.  QG > 64 returns UQ_ERR_INVALID_ARG.
 * Device preconditions: 0 <= seq_lens[b] <= max_seq_len (larger values are clamped to
 * max_seq_len); block_table[b][t / block_size] in [0, num_blocks) for every t < L_b;
 * entries past a sequence's last block are never read; slot bytes of tokens t >= L_b are
 * never used (they may hold anything, NaN codes included). */
int uq_paged_decode(const void* query, int q_dtype, int64_t q_stride_seq,
                    int64_t q_stride_head, const uint8_t* kv_cache, int64_t num_blocks,
                    int32_t block_size, int32_t num_kv_heads, int32_t slot_bytes,
                    int kv_format, const float* k_scale, const float* v_scale,
                    const int8_t* rot_signs, const int32_t* block_table, int32_t bt_stride,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                    int32_t head_dim, int32_t max_seq_len, float softmax_scale,
                    int32_t num_partitions, void* part_out, float* part_max,
                    float* part_sum, void* stream);

/* uq_paged_reduce -- flash-combine of the partials of uq_paged_decode ([P3] partition
 * split + parallel reduce; empty-partition handling).  For every (b, h, g), over the
 * partitions p < n_b = min(P, ceil(L_b / 256)) with l_p > 0:
 *   M = max_p m_p,  w_p = l_p exp(m_p - M),  out = sum_p w_p o_p / sum_p w_p
 * and out = 0 when there is none.  Partial rows of partitions with l_p = 0 are not
 * read (their bytes may be anything).
 *   part_out / part_max / part_sum   as written by uq_paged_decode (same shapes and P)
 *   out        [num_seqs, num_kv_heads * qg, head_dim] of out_dtype (UQ_F32 or UQ_BF16;
 *              the query dtype, [P3] output dtype follows the query), element strides
 *              o_stride_seq / o_stride_head (head dim contiguous).
 * Supported: head_dim in {128, 256}, 1 <= qg <= 64. */
int uq_paged_reduce(const void* part_out, const float* part_max, const float* part_sum,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                    int32_t qg, int32_t head_dim, int32_t num_partitions,
                    int32_t max_seq_len, void* out, int out_dtype, int64_t o_stride_seq,
                    int64_t o_stride_head, void* stream);

/* uq_paged_decode_mtp -- uq_paged_decode for query_len >= 1 query rows per sequence
 * (multi-token decode, [P3] MTP path with query_length > 1).  Query row j of sequence b
 * sees the tokens t < L_b - query_len + 1 + j ([P3] causal window of each query row: the
 * last row sees the whole sequence); a row that sees no token of a partition leaves that
 * partition empty for the row (m = -inf, l = 0), and a row that sees no token at all
 * reduces to 0.  Arguments as uq_paged_decode, except:
 *   query         [num_seqs * query_len, num_q_heads, head_dim]; row b*query_len + j is
 *                 query j of sequence b; q_stride_seq is the stride between query rows.
 *   part_out      bf16 [num_seqs, num_kv_heads, P, query_len * QG, head_dim]
 *   part_max,     f32  [num_seqs, num_kv_heads, P, query_len * QG]; row j*QG + g holds
 *   part_sum      query j, head h*QG + g (uq_decode_workspace_bytes with qg = query_len*QG)
 * Supported: fp8 with query_len * QG <= 64 (one pass over the cache per 16 rows), fp4
 * with query_len * QG <= 16; query_len = 1 is exactly uq_paged_decode.  query_len < 1
 * returns UQ_ERR_INVALID_ARG. */
int uq_paged_decode_mtp(const void* query, int q_dtype, int64_t q_stride_seq,
                        int64_t q_stride_head, const uint8_t* kv_cache, int64_t num_blocks,
                        int32_t block_size, int32_t num_kv_heads, int32_t slot_bytes,
                        int kv_format, const float* k_scale, const float* v_scale,
                        const int8_t* rot_signs, const int32_t* block_table, int32_t bt_stride,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t query_len,
                        int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                        float softmax_scale, int32_t num_partitions, void* part_out,
                        float* part_max, float* part_sum, void* stream);

/* uq_paged_reduce_mtp -- uq_paged_reduce of the partials of uq_paged_decode_mtp: for
 * every (b, j, h, g) the flash-combine above over the partitions with l_p > 0 of partial
 * row j*qg + g, written to out row b*query_len + j, head h*qg + g.
 *   out        [num_seqs * query_len, num_kv_heads * qg, head_dim]; o_stride_seq is the
 *              stride between query rows.
 * Supported: head_dim in {128, 256}, query_len >= 1, qg >= 1, query_len * qg <= 64. */
int uq_paged_reduce_mtp(const void* part_out, const float* part_max, const float* part_sum,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_kv_heads,
                        int32_t query_len, int32_t qg, int32_t head_dim, int32_t num_partitions,
                        int32_t max_seq_len, void* out, int out_dtype, int64_t o_stride_seq,
                        int64_t o_stride_head, void* stream);

/* uq_paged_attention -- one whole decode step: uq_paged_decode_mtp and the flash-combine
 * of uq_paged_reduce_mtp ([P3] partition split + parallel reduce) in one call, writing
 * the attention output directly.  The result is that of the two calls in sequence:
 *   out[b*query_len + j, h*QG + g, :] = v_scale * sum_t exp(s_t - M) v_t / sum_t exp(s_t - M)
 * over the tokens t the query row sees (0 when it sees none), in the query dtype.
 * Arguments as uq_paged_decode_mtp, except that the partial buffers are replaced by:
 *   workspace       device buffer of workspace_bytes >= uq_attention_workspace_bytes(...)
 *                   for the same sizes, 256-byte aligned.  It must be zero-filled once
 *                   before its first use (e.g. hipMemset after allocating it); every
 *                   call that completes leaves it fit for the next call of any sizes
 *                   that fit it (its first 256 KiB hold arrival counters, which
 *                   every call leaves at zero and nothing else writes), so it can be
 *                   reused across calls and graph replays.  Calls that overlap in time
 *                   on one workspace race.
 *   out             [num_seqs * query_len, num_q_heads, head_dim] of q_dtype, element
 *                   strides o_stride_seq / o_stride_head (> 0, 16-byte multiples; the head
 *                   dim is contiguous, out 16-byte aligned).
 * How it runs: with the fp8 formats and head groups (num_kv_heads a multiple of 4, or of
 * 2 for groups of 33-64 rows) one launch; every work unit of a (sequence, kv
 * head) that does not cover the whole sequence leaves its softmax state in the workspace
 * and counts its partitions with a device-scope atomic, and the unit that completes the
 * count merges the states, in a fixed order whichever unit finishes last, and writes the
 * output rows.  Other formats and head counts run the decode into partials held in the
 * workspace, then the reduce (two launches).  Either way the output depends only on the
 * inputs: repeated calls give bit-identical results.  Errors
 * as uq_paged_decode_mtp, plus UQ_ERR_INVALID_ARG for a NULL, misaligned or too small
 * workspace or output. */
int uq_paged_attention(const void* query, int q_dtype, int64_t q_stride_seq,
                       int64_t q_stride_head, const uint8_t* kv_cache, int64_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t slot_bytes,
                       int kv_format, const float* k_scale, const float* v_scale,
                       const int8_t* rot_signs, const int32_t* block_table, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t query_len,
                       int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                       float softmax_scale, int32_t num_partitions, void* workspace,
                       size_t workspace_bytes, void* out, int64_t o_stride_seq,
                       int64_t o_stride_head, void* stream);

/* uq_index_score -- nvfp4 index scores ([P2] compile_score_decode).  For request r,
 * query row j < query_len, index head h and page b < ceil(L_r / 128):
 *   scores[h, r*QL + j, b] = max over tokens t of page b with t <= L_r - QL + j of
 *                            sum_d q[r*QL + j, h, d] * k[t, d]
 * with k = e2m1(code) * e4m3(scale of its 16-dim group), products exact and fp32
 * accumulation; -inf when page b holds no such token ([P2] frag_max / score_cgs).
 *   q        e4m3 codes [num_reqs*query_len, heads, head_dim], byte strides
 *            q_stride_tok / q_stride_head (> 0, multiples of 16; dims contiguous).  One
 *            request's rows, (query_len - 1) * q_stride_tok + (heads - 1) * q_stride_head
 *            + head_dim bytes, must span less than 2^31 (else UQ_ERR_UNSUPPORTED).
 *   k_pages  [num_pages] pages of page_stride bytes: codes [128 tok][head_dim/2] then
 *            scales [128 tok][head_dim/16] ([P2] load_tile offsets).  page_stride >=
 *            128 * (head_dim/2 + head_dim/16) and a multiple of 16.
 *   block_table [num_reqs, bt_stride] int32 page ids; seq_lens [num_reqs] int32.
 *   scores   fp32 [heads, num_reqs*query_len, max_blocks], element strides s_stride_head,
 *            s_stride_row (page index contiguous).  Cells with b >= ceil(L_r/128) (or
 *            b >= max_blocks) are not written.  s_stride_row >= max_blocks, and with
 *            heads > 1 the heads' planes may not overlap: s_stride_head >=
 *            (num_reqs*query_len - 1) * s_stride_row + max_blocks (else
 *            UQ_ERR_INVALID_ARG).
 *   init_blocks, local_blocks: sentinel block counts of [P2] block_sentinels; their
 *            semantics are not given on the page, so both must be 0.
 * Supported: head_dim 128, heads in {1, 2, 4}, 1 <= heads*query_len <= 32.
 * Device preconditions: query_len <= seq_lens[r]; page ids of visible pages in
 * [0, num_pages). */
int uq_index_score(const uint8_t* q, int64_t q_stride_tok, int64_t q_stride_head,
                   const uint8_t* k_pages, int64_t page_stride, int64_t num_pages,
                   const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                   int32_t num_reqs, int32_t query_len, int32_t heads, int32_t head_dim,
                   int32_t init_blocks, int32_t local_blocks, float* scores,
                   int64_t s_stride_head, int64_t s_stride_row, int32_t max_blocks,
                   void* stream);

/* Bytes of the three uq_paged_decode partial buffers together (part_out + part_max +
 * part_sum), each rounded up to 256 bytes; 0 on invalid sizes.  Host-only. */
size_t uq_decode_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t qg,
                                 int32_t head_dim, int32_t num_partitions);

/* uq_paged_attention_noalloc -- uq_paged_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, arguments and results, without the workspace argument.  Its
 * workspace is a 64 MiB array in the library's device data (one copy per GPU, held until
 * the process ends); the library allocates nothing.  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (two streams, two threads) race.  The
 * counters in its first 256 KiB start at zero and every completed call leaves them at
 * zero; nothing else is written there.
 * A call whose uq_attention_workspace_bytes exceeds 64 MiB returns UQ_ERR_INVALID_ARG
 * before launching anything (use uq_paged_attention); other errors as uq_paged_attention. */
int uq_paged_attention_noalloc(const void* query, int q_dtype, int64_t q_stride_seq,
                               int64_t q_stride_head, const uint8_t* kv_cache,
                               int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                               int32_t slot_bytes, int kv_format, const float* k_scale,
                               const float* v_scale, const int8_t* rot_signs,
                               const int32_t* block_table, int32_t bt_stride,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t query_len,
                               int32_t num_q_heads, int32_t head_dim, int32_t max_seq_len,
                               float softmax_scale, int32_t num_partitions, void* out,
                               int64_t o_stride_seq, int64_t o_stride_head, void* stream);

/* Bytes of the uq_paged_attention workspace for these sizes on the current device (the
 * work decomposition depends on its compute-unit count); 0 on invalid sizes.  Host-only. */
size_t uq_attention_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t query_len,
                                    int32_t qg, int32_t head_dim, int32_t num_partitions,
                                    int32_t max_seq_len, int kv_format);

/* Text describing the last non-OK return on the calling thread ("" if none).  The
 * string is owned by the library and valid until the next call on this thread. */
const char* uq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* UQ_PAGED_H */

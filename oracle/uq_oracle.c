/*
 * uq_oracle.c -- plain fp64 CPU oracle for quantized paged-attention decode and for
 * the nvfp4 index scorer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is compiled into liboracle.so and is called
 * from the tests, from the package's smoke check and from the CPU-baseline leg of the
 * benchmark.  The HIP library never links, includes or calls it, and it includes
 * nothing from the HIP library.
 *
 * Everything here is written to be checked by eye against the pages:
 *   [P1] "ultraquant_decode_hd256" (vLLM PR 59857 API page): FP4 D=256 decode kernel,
 *        its slot layout (builder docstring and the K/V scale/code offset constants),
 *        partition -> tile-group map (builder comments, STEP F trip count), the
 *        Walsh-Hadamard query rotation (STEP B'), masking and online softmax (STEP F),
 *        and the partition epilogue (STEP G).
 *   [P2] "nvfp4_index_decode/kernel" (vLLM PR 59747 API page): compile_score_decode --
 *        page layout (load_tile), per-page max of q.k (frag_max) and the causal limit
 *        of trailing query rows (score_cgs).
 *   [P3] ROCm/FlyDSL PR #825 "pa_decode_tile": per-tensor fp8 K/V decode, partition
 *        split + flash-combine reduce, empty-partition handling (l = 0 -> 1).
 *
 * Arithmetic is fp64 throughout; codes are decoded by closed-form formulas (no tables),
 * and attention is a direct two-pass masked softmax over every visible token -- no
 * blocking, no online rescaling, no fusion.
 *
 * Parity pins: every function here is pinned by tests that do not re-type its formula
 * (exhaustive code tables against the OCP specification anchors and torch's float8
 * cast, torch's scaled_dot_product_attention on gathered dense K/V, single-token and
 * equal-score invariants, one-hot gathers, partition and permutation invariance, a
 * butterfly WHT, and a brute-force per-page max).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops below run on (1 when built without OpenMP). */
int uqo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

#define UQO_FMT_FP8_E4M3 0       /* slot: K e4m3[D] | V e4m3[D]                          */
#define UQO_FMT_FP4_E4M3S 1      /* slot: Kc[D/2] | Ks[D/32] | Vc[D/2] | Vs[D/32], e4m3 s */
#define UQO_FMT_FP4_UE8M0S 2     /* same slot, UE8M0 group scales ([P1] STEP F V path)    */
#define UQO_FMT_FP8_E4M3_TOK 3   /* fp8 slot, one f32 K and V scale per (block, head, pos) */

#define UQO_TILE_GROUP 256       /* tokens per tile-group: 16 tiles of 16 ([P1] STEP F)    */
#define UQO_INDEX_PAGE 128       /* tokens per index page ([P2] kernel argument comments)  */

/* ---------------------------------------------------------------- codecs ------------ */

/* OCP FP8 E4M3FN: sign, 4-bit exponent (bias 7), 3-bit mantissa.  Exponent 0 is
 * subnormal (m * 2^-9); S.1111.111 is NaN; there is no infinity.  gfx950 decodes this
 * format ([P3] review notes: gfx942 uses FNUZ, gfx950 OCP e4m3fn). */
double uqo_e4m3(uint32_t byte) {
  const int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp((double)(8 + m), e - 10);
  return s ? -mag : mag;
}

/* OCP FP4 E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa.
 * Magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}. */
double uqo_e2m1(uint32_t nibble) {
  const int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, m = nibble & 1;
  double mag;
  if (e == 0)
    mag = 0.5 * m;
  else
    mag = ldexp((double)(2 + m), e - 2);
  return s ? -mag : mag;
}

/* UE8M0 group scale 2^(byte-127); byte 0 is the zero sentinel of [P1] (STEP F, scale
 * words: "byte==0 -> +0.0"); byte 255 is NaN. */
double uqo_ue8m0(uint32_t byte) {
  if (byte == 0) return 0.0;
  if (byte == 255) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* Element d of a packed e2m1 vector: element 2i is the low nibble of byte i, element
 * 2i+1 the high nibble ([P1] V dequant: "srcSel s picks byte s of the word (nibbles
 * 2s, 2s+1)"). */
static double e2m1_at(const uint8_t* codes, int d) {
  const uint8_t b = codes[d >> 1];
  return uqo_e2m1((d & 1) ? (b >> 4) : (b & 15));
}

/* Bytes of slot content for a format and head dim (0 if unsupported). */
int uqo_slot_content_bytes(int kv_format, int head_dim) {
  if (kv_format == UQO_FMT_FP8_E4M3 || kv_format == UQO_FMT_FP8_E4M3_TOK) return 2 * head_dim;
  if (kv_format == UQO_FMT_FP4_E4M3S || kv_format == UQO_FMT_FP4_UE8M0S) {
    if (head_dim % 32) return 0;
    return 2 * (head_dim / 2 + head_dim / 32);
  }
  return 0;
}

/* Decode one (token, head) slot into k[D] and v[D] (unscaled by the per-tensor fp8
 * scales).  fp4 slot layout of [P1] (builder docstring and the K_SCALES / V_CODES /
 * V_SCALES offset constants): K codes [0, D/2), K group scales [D/2, D/2 + D/32),
 * V codes next, V group scales last; one scale per 32 consecutive dims. */
static void decode_slot(const uint8_t* slot, int kv_format, int D, double* k, double* v) {
  if (kv_format == UQO_FMT_FP8_E4M3 || kv_format == UQO_FMT_FP8_E4M3_TOK) {
    for (int d = 0; d < D; ++d) {
      k[d] = uqo_e4m3(slot[d]);
      v[d] = uqo_e4m3(slot[D + d]);
    }
    return;
  }
  const uint8_t* kc = slot;
  const uint8_t* ks = slot + D / 2;
  const uint8_t* vc = ks + D / 32;
  const uint8_t* vs = vc + D / 2;
  for (int d = 0; d < D; ++d) {
    const int g = d / 32;
    const double sk = kv_format == UQO_FMT_FP4_E4M3S ? uqo_e4m3(ks[g]) : uqo_ue8m0(ks[g]);
    const double sv = kv_format == UQO_FMT_FP4_E4M3S ? uqo_e4m3(vs[g]) : uqo_ue8m0(vs[g]);
    k[d] = e2m1_at(kc, d) * sk;
    v[d] = e2m1_at(vc, d) * sv;
  }
}

/* ------------------------------------------------------------ rotation -------------- */

/* Query rotation of [P1] STEP B': q' = (q * s) H / sqrt(D), H the Sylvester Hadamard
 * matrix H[i][j] = (-1)^popcount(i & j), s the +-1 sign diagonal.  Written as the
 * direct O(D^2) sum, not a butterfly.  D must be a power of two. */
void uqo_rotate(const double* q, const int8_t* signs, int D, double* out) {
  const double inv = 1.0 / sqrt((double)D);
  for (int j = 0; j < D; ++j) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) {
      const double h = (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
      acc += q[i] * (double)signs[i] * h;
    }
    out[j] = acc * inv;
  }
}

/* ------------------------------------------------------------ decode ---------------- */

/* Paged decode attention, fp64, for query_len (QL) query rows per sequence.
 *
 * q        : [B * QL, Hq, D] widened to fp64, element strides q_ss (query row), q_sh
 *            (head); row b * QL + j is query j of sequence b
 * cache    : [num_blocks, block_size, Hk, slot_bytes] bytes
 * bt       : [B, bt_stride] int32 physical block ids; only entries for visible tokens
 *            (t < seq_lens[b]) are read
 * rot      : NULL, or +-1 signs of the query rotation (fp4 formats)
 * Per (b, j, h, g) with Hq = Hk * QG and head index h*QG + g, query j sees the tokens
 * t < L_bj = L_b - QL + 1 + j (the last query row sees the whole sequence: [P3] MTP
 * causal window of each query row):
 *   s_t = softmax_scale * k_scale * (q' . k_t)   for every t < L_bj
 *   out = v_scale * sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s)
 * A row with L_bj <= 0 is zero.  QL = 1 is single-token decode.
 *
 * Per-token fp8 scales (kv_format UQO_FMT_FP8_E4M3_TOK, [P3] per_token_kv mode): the
 * slot holds the same e4m3 K and V codes, and token t of a sequence, in physical block
 * blk at position t mod block_size, has the decoded values
 *   k_t = e4m3(K codes) * k_tok[(blk * Hk + h) * block_size + t mod block_size]
 *   v_t = e4m3(V codes) * v_tok[(blk * Hk + h) * block_size + t mod block_size]
 * (f32 scale tensors [num_blocks, Hk, block_size]); the per-tensor k_scale and v_scale
 * still multiply on top (the binding passes 1 for them).  Other formats ignore k_tok and
 * v_tok.
 *
 * If num_partitions > 0 the per-partition statistics are also produced.  Partition p
 * owns the 256-token tile-groups p, p+P, p+2P, ... ([P1] builder comment on the strided
 * map and STEP F trip count); over its visible tokens:
 *   part_m = max s_t,  part_l = sum exp(s_t - part_m),
 *   part_o = v_scale * sum exp(s_t - part_m) v_t / part_l
 * and an empty partition is (m = -inf, l = 0, o = 0) ([P1] STEP G; [P3] empty-partition
 * fix).  Layouts: part_o [B, Hk, P, QL*QG, D], part_m / part_l [B, Hk, P, QL*QG], row
 * j*QG + g; out [B * QL, Hq, D].
 *
 * Returns 0, or -1 if a visible token's block id is outside [0, num_blocks), or -2 on
 * bad sizes. */
int uqo_decode_q(const double* q, int64_t q_ss, int64_t q_sh, const uint8_t* cache,
                 int64_t num_blocks, int block_size, int num_kv_heads, int slot_bytes,
                 int kv_format, double k_scale, double v_scale, const float* k_tok,
                 const float* v_tok, const int8_t* rot,
                 const int32_t* bt, int bt_stride, const int32_t* seq_lens, int num_seqs,
                 int query_len, int num_q_heads, int head_dim, double softmax_scale,
                 double* out, int num_partitions, double* part_m, double* part_l,
                 double* part_o) {
  const int B = num_seqs, Hk = num_kv_heads, D = head_dim, QL = query_len;
  if (Hk <= 0 || num_q_heads % Hk != 0 || D <= 0 || block_size <= 0 || QL < 1) return -2;
  const int QG = num_q_heads / Hk;
  const int QR = QL * QG; /* partial rows per (sequence, kv head) */
  const int P = num_partitions;
  if (slot_bytes < uqo_slot_content_bytes(kv_format, D) ||
      uqo_slot_content_bytes(kv_format, D) == 0)
    return -2;
  if (kv_format == UQO_FMT_FP8_E4M3_TOK && (!k_tok || !v_tok)) return -2;
  int status = 0;

#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < Hk; ++h) {
      const int Lseq = seq_lens[b];
      double* K = (double*)malloc(sizeof(double) * (size_t)(Lseq > 0 ? Lseq : 1) * D);
      double* V = (double*)malloc(sizeof(double) * (size_t)(Lseq > 0 ? Lseq : 1) * D);
      double* s = (double*)malloc(sizeof(double) * (size_t)(Lseq > 0 ? Lseq : 1));
      double* qr = (double*)malloc(sizeof(double) * D);
      double* qv = (double*)malloc(sizeof(double) * D);
      int bad = 0;
      /* gather and decode every visible token of this (sequence, kv head) */
      for (int t = 0; t < Lseq && !bad; ++t) {
        const int64_t blk = bt[(int64_t)b * bt_stride + t / block_size];
        if (blk < 0 || blk >= num_blocks) {
          bad = 1;
          break;
        }
        const int64_t slot_index = (blk * block_size + t % block_size) * Hk + h;
        decode_slot(cache + slot_index * slot_bytes, kv_format, D, K + (size_t)t * D,
                    V + (size_t)t * D);
        if (kv_format == UQO_FMT_FP8_E4M3_TOK) {
          const int64_t si = (blk * Hk + h) * block_size + t % block_size;
          const double sk = k_tok[si], sv = v_tok[si];
          for (int d = 0; d < D; ++d) {
            K[(size_t)t * D + d] *= sk;
            V[(size_t)t * D + d] *= sv;
          }
        }
      }
      if (bad) {
#pragma omp atomic write
        status = -1;
      }
      for (int r = 0; r < QR && !bad; ++r) {
        const int j = r / QG, g = r % QG;
        /* the tokens this query row sees */
        const int L = Lseq - QL + 1 + j > 0 ? Lseq - QL + 1 + j : 0;
        const int qh = h * QG + g;
        const int64_t qrow = (int64_t)b * QL + j;
        for (int d = 0; d < D; ++d) qv[d] = q[qrow * q_ss + (int64_t)qh * q_sh + d];
        if (rot)
          uqo_rotate(qv, rot, D, qr);
        else
          memcpy(qr, qv, sizeof(double) * D);
        /* scores */
        for (int t = 0; t < L; ++t) {
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += qr[d] * K[(size_t)t * D + d];
          s[t] = softmax_scale * k_scale * dot;
        }
        /* full softmax over all visible tokens */
        double* o = out + (qrow * num_q_heads + qh) * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (L > 0) {
          double mx = -INFINITY;
          for (int t = 0; t < L; ++t) mx = s[t] > mx ? s[t] : mx;
          double den = 0.0;
          for (int t = 0; t < L; ++t) {
            const double w = exp(s[t] - mx);
            den += w;
            for (int d = 0; d < D; ++d) o[d] += w * V[(size_t)t * D + d];
          }
          for (int d = 0; d < D; ++d) o[d] = v_scale * o[d] / den;
        }
        /* per-partition statistics: partition p holds tile-groups p, p+P, p+2P, ... */
        for (int p = 0; p < P; ++p) {
          const int64_t ml = (((int64_t)b * Hk + h) * P + p) * QR + r;
          double* po = part_o + ml * D;
          double mx = -INFINITY, den = 0.0;
          int any = 0;
          for (int d = 0; d < D; ++d) po[d] = 0.0;
          for (int tg = p; (int64_t)tg * UQO_TILE_GROUP < L; tg += P) {
            for (int t = tg * UQO_TILE_GROUP; t < (tg + 1) * UQO_TILE_GROUP && t < L; ++t) {
              any = 1;
              mx = s[t] > mx ? s[t] : mx;
            }
          }
          if (!any) {
            part_m[ml] = -INFINITY;
            part_l[ml] = 0.0;
            continue;
          }
          for (int tg = p; (int64_t)tg * UQO_TILE_GROUP < L; tg += P) {
            for (int t = tg * UQO_TILE_GROUP; t < (tg + 1) * UQO_TILE_GROUP && t < L; ++t) {
              const double w = exp(s[t] - mx);
              den += w;
              for (int d = 0; d < D; ++d) po[d] += w * V[(size_t)t * D + d];
            }
          }
          for (int d = 0; d < D; ++d) po[d] = v_scale * po[d] / den;
          part_m[ml] = mx;
          part_l[ml] = den;
        }
      }
      free(K);
      free(V);
      free(s);
      free(qr);
      free(qv);
    }
  }
  return status;
}

int uqo_decode(const double* q, int64_t q_ss, int64_t q_sh, const uint8_t* cache,
               int64_t num_blocks, int block_size, int num_kv_heads, int slot_bytes,
               int kv_format, double k_scale, double v_scale, const int8_t* rot,
               const int32_t* bt, int bt_stride, const int32_t* seq_lens, int num_seqs,
               int num_q_heads, int head_dim, double softmax_scale, double* out,
               int num_partitions, double* part_m, double* part_l, double* part_o) {
  return uqo_decode_q(q, q_ss, q_sh, cache, num_blocks, block_size, num_kv_heads, slot_bytes,
                      kv_format, k_scale, v_scale, NULL, NULL, rot, bt, bt_stride, seq_lens,
                      num_seqs, 1,
                      num_q_heads, head_dim, softmax_scale, out, num_partitions, part_m,
                      part_l, part_o);
}

/* Flash-combine ([P3] partition split + parallel reduce): for each (b, j, h, g),
 *   M = max_p part_m,  w_p = part_l * exp(part_m - M),
 *   out = sum_p w_p part_o / sum_p w_p
 * over the partitions p < min(P, ceil(L_b / 256)) that hold tokens of the row (l > 0); a
 * row with no tokens is zero.  Partials use the layouts of uqo_decode_q (rows j*QG + g);
 * out is [B * QL, Hk*QG, D]. */
void uqo_reduce_q(const double* part_o, const double* part_m, const double* part_l,
                  const int32_t* seq_lens, int num_seqs, int num_kv_heads, int query_len,
                  int qg, int head_dim, int num_partitions, double* out) {
  const int Hk = num_kv_heads, QL = query_len, QG = qg, D = head_dim, P = num_partitions;
  const int QR = QL * QG;
  for (int b = 0; b < num_seqs; ++b) {
    const int L = seq_lens[b];
    const int ntg = (L + UQO_TILE_GROUP - 1) / UQO_TILE_GROUP;
    const int n = ntg < P ? ntg : P;
    for (int h = 0; h < Hk; ++h) {
      for (int r = 0; r < QR; ++r) {
        const int j = r / QG, g = r % QG;
        double* o = out + (((int64_t)b * QL + j) * Hk * QG + h * QG + g) * D;
        double M = -INFINITY;
        for (int p = 0; p < n; ++p) {
          const double m = part_m[(((int64_t)b * Hk + h) * P + p) * QR + r];
          M = m > M ? m : M;
        }
        double den = 0.0;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (n == 0) continue;
        for (int p = 0; p < n; ++p) {
          const int64_t ml = (((int64_t)b * Hk + h) * P + p) * QR + r;
          if (part_l[ml] == 0.0) continue; /* no tokens of this row */
          const double w = part_l[ml] * exp(part_m[ml] - M);
          den += w;
          for (int d = 0; d < D; ++d) o[d] += w * part_o[ml * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] = den > 0.0 ? o[d] / den : 0.0;
      }
    }
  }
}

void uqo_reduce(const double* part_o, const double* part_m, const double* part_l,
                const int32_t* seq_lens, int num_seqs, int num_kv_heads, int qg, int head_dim,
                int num_partitions, double* out) {
  uqo_reduce_q(part_o, part_m, part_l, seq_lens, num_seqs, num_kv_heads, 1, qg, head_dim,
               num_partitions, out);
}

/* ------------------------------------------------------------ index scorer ---------- */

/* nvfp4 index scores of [P2].
 *
 * q      : e4m3 codes [num_reqs * QL, H, D], byte strides q_st (token), q_sh (head)
 * pages  : [num_pages] pages of page_stride bytes; a page holds 128 tokens as
 *          codes [128][D/2] (e2m1, low nibble first) then scales [128][D/16] (e4m3,
 *          one per 16 dims) ([P2] load_tile: codes at t*1024, scales after the
 *          8192-byte code region)
 * bt     : [num_reqs, bt_stride] int32 page ids; only pages b < ceil(L_r/128) are read
 * scores : fp32-valued output widened to fp64 here, [H, num_reqs*QL, *] element strides
 *          s_sh (head), s_st (row); column b is page b
 * For request r, query row j < QL, head h, page b < ceil(L_r / 128):
 *   scores[h, r*QL + j, b] = max over tokens t of page b with t <= L_r - QL + j of
 *                            sum_d q[r*QL + j, h, d] * k[t, d]
 * (-inf if the page holds no such token; [P2] score_cgs causal limit).  Every other cell
 * is left as it was.  Returns 0, or -1 on a page id outside [0, num_pages). */
int uqo_index_score(const uint8_t* q, int64_t q_st, int64_t q_sh, const uint8_t* pages,
                    int64_t page_stride, int64_t num_pages, const int32_t* bt, int bt_stride,
                    const int32_t* seq_lens, int num_reqs, int query_len, int heads,
                    int head_dim, double* scores, int64_t s_sh, int64_t s_st) {
  const int QL = query_len, H = heads, D = head_dim;
  const int code_bytes = D / 2, scale_bytes = D / 16;
  int status = 0;
#pragma omp parallel for schedule(dynamic)
  for (int r = 0; r < num_reqs; ++r) {
    const int L = seq_lens[r];
    const int nblk = (L + UQO_INDEX_PAGE - 1) / UQO_INDEX_PAGE;
    double* k = (double*)malloc(sizeof(double) * D);
    double* qv = (double*)malloc(sizeof(double) * D);
    for (int b = 0; b < nblk; ++b) {
      const int64_t page = bt[(int64_t)r * bt_stride + b];
      if (page < 0 || page >= num_pages) {
#pragma omp atomic write
        status = -1;
        break;
      }
      const uint8_t* pg = pages + page * page_stride;
      for (int j = 0; j < QL; ++j) {
        const int64_t row = (int64_t)r * QL + j;
        const int64_t lim = (int64_t)L - QL + j; /* last visible token of this row */
        for (int h = 0; h < H; ++h) {
          for (int d = 0; d < D; ++d) qv[d] = uqo_e4m3(q[row * q_st + h * q_sh + d]);
          double best = -INFINITY;
          for (int i = 0; i < UQO_INDEX_PAGE; ++i) {
            const int64_t t = (int64_t)b * UQO_INDEX_PAGE + i;
            if (t > lim) break;
            const uint8_t* codes = pg + (int64_t)i * code_bytes;
            const uint8_t* sc = pg + (int64_t)UQO_INDEX_PAGE * code_bytes + (int64_t)i * scale_bytes;
            for (int d = 0; d < D; ++d) k[d] = e2m1_at(codes, d) * uqo_e4m3(sc[d / 16]);
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += qv[d] * k[d];
            best = dot > best ? dot : best;
          }
          scores[h * s_sh + row * s_st + b] = best;
        }
      }
    }
    free(k);
    free(qv);
  }
  return status;
}

/*
 * pkv_oracle.c -- plain CPU oracle for paged-KV attention (TEST INFRASTRUCTURE).
 *
 * This file is the parity reference for the HIP library.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the product
 * path never calls it.  It shares no code, header or constant with the HIP
 * sources.  It is deliberately slow: single-threaded, fp64 throughout, one
 * (query row, head) at a time, every KV element decoded from its storage bits
 * at the point of use.
 *
 * What it computes (the plain definition the paged kernels must reach):
 *
 *   For request b with n_b query rows (rows q_indptr[b] .. q_indptr[b+1]) and
 *   total KV length L_b = seq_lens[b] (which counts the request's own query
 *   rows), query row i (0 <= i < n_b) of head h attends keys j in [0, c) with
 *       c = L_b - n_b + i + 1   when causal   (inclusive bound L_b - n_b + i)
 *       c = L_b                 otherwise.
 *   Key j lives at offset j mod P of page block_tables[b][j / P]           (A)
 *   KV head g = h / (Hq / Hkv)  (query heads grouped contiguously)         (B)
 *       s_j   = scale * k_scale * sum_d q[d] * k_j[d]
 *       m     = max_j s_j ,  w_j = exp(s_j - m),  l = sum_j w_j
 *       out   = v_scale * sum_j w_j v_j / l ,      lse = m + ln l
 *   Rows with no visible key (c <= 0) give out = 0 and lse = -inf.
 *   Attention sinks (optional, one logit sigma_h per query head, in the units
 *   of s_j): the softmax denominator gains exp(sigma_h) and no value, i.e.
 *       lse' = ln(exp(lse) + exp(sigma_h)),  out' = out * exp(lse - lse')
 *   (an empty row gets lse' = sigma_h and out' = 0); the Split-KV partials
 *   carry no sink, the merge applies it once.                              (C)
 *   Separate K and V page tables (optional): key j is read through k_table,
 *   value j through v_table.                                               (D)
 *
 * Passages followed:
 *   (A) flashinfer.cake_fmha API page: the paged decode call takes query,
 *       kv_cache, block_tables, seq_lens and max_kv_len; PR #5952 page
 *       summary: a dense [B, max_pages] page table.
 *   (B) flashinfer.cake_fmha API page, FP8 qualification paragraph: GQA
 *       group size eight; the head->group map itself is not stated, the
 *       contiguous grouping is the reading taken here.
 *   Causal bound: PR #4557 page, the review comment that flags an exclusive
 *       causal bound as a critical bug, and the test-reference comment that
 *       slices the gathered keys up to and including seq_len - q_len + i:
 *       the bound is inclusive.
 *   seq_lens counts the appended rows: PR #5956 section "Contract" (the
 *       length is the request's total once the new rows are in the cache).
 *   Scales: bmm1_scale / bmm2_scale arguments (PR #4557 page, MLA dispatcher
 *       excerpt) and the FP8 storage rule stored = x / scale (PR #5956
 *       section "Contract"): the logit scale is scale*k_scale, the output carries
 *       v_scale.
 *   MLA: PR #4557 page, V is the 512 latent channels of the shared 576-wide
 *       row; expressed here by passing the K pool again as the V pool with a
 *       smaller head_dim_v.
 *   (C) The pages list `sinks` among the decode call's arguments (PR #4557
 *       page, MLA dispatcher excerpt and the benchmark row "B1 KV1024 page64
 *       sink") without defining them; the reading taken is one extra logit
 *       per query head in the softmax denominator, with no value row.
 *   (D) flashinfer.cake_fmha API page, BF16 context profiles: a q257/KV1024
 *       profile with separate K/V page tables.
 *   Split-KV + log-sum-exp merge: PR #4557 page (Split-KV reduction, split8
 *       reducer with 32 statistics slots, two-kernel split-major ABI).  The
 *       oracle's split mode partitions [0, c) at page-aligned boundaries and
 *       merges with  L* = max_s lse_s,  w_s = exp(lse_s - L*),
 *       out = sum_s w_s O_s / sum_s w_s,  lse = L* + ln sum_s w_s.
 *
 * Element decoding (from the format definitions, not from any library):
 *   fp32 as is; bf16 = the 16 high bits of an fp32; OCP e4m3 ("fn"): sign,
 *   4-bit exponent with bias 7, 3-bit mantissa, exponent 0 is subnormal
 *   2^-6 * M/8, 0x7F / 0xFF are NaN, no infinities, max finite 448.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3 = 2 };

typedef struct {
  int32_t batch;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim_qk;
  int32_t head_dim_v;
  int32_t page_size;
  int32_t causal;
  int32_t q_dtype;
  int32_t k_dtype;
  int32_t v_dtype;
  const int32_t* q_indptr;   /* [batch + 1] */
  const int32_t* seq_lens;   /* [batch] */
  const int32_t* k_table;    /* [batch, table_stride] */
  const int32_t* v_table;    /* [batch, table_stride] */
  int64_t table_stride;
  const void* q;             /* [T_q, Hq, D_qk], contiguous */
  const void* k;
  const void* v;
  int64_t k_page_stride, k_head_stride, k_tok_stride; /* in elements */
  int64_t v_page_stride, v_head_stride, v_tok_stride;
  double scale, k_scale, v_scale;
  const double* sinks;       /* [num_qo_heads] or NULL: no sink */
} orc_problem;

double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

double orc_e4m3_to_double(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

static double load_elem(const void* base, int dtype, int64_t idx) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[idx]);
    case ORC_E4M3: return orc_e4m3_to_double(((const uint8_t*)base)[idx]);
  }
  return NAN;
}

/* locate the request that owns global query row t */
static int find_request(const orc_problem* p, int64_t t) {
  for (int b = 0; b < p->batch; ++b)
    if (t >= p->q_indptr[b] && t < p->q_indptr[b + 1]) return b;
  return -1;
}

/* number of visible keys for query row t of request b */
static int64_t visible_keys(const orc_problem* p, int b, int64_t t) {
  int64_t n = p->q_indptr[b + 1] - p->q_indptr[b];
  int64_t i = t - p->q_indptr[b];
  int64_t L = p->seq_lens[b];
  int64_t c = p->causal ? L - n + i + 1 : L;
  if (c > L) c = L;
  return c;
}

static int64_t key_offset(int64_t page, int64_t g, int64_t tok, int64_t ps, int64_t hs, int64_t ts) {
  return page * ps + g * hs + tok * ts;
}

/* logit of key j for (row t, head h) */
static double logit(const orc_problem* p, int b, int64_t t, int h, int64_t j) {
  int G = p->num_qo_heads / p->num_kv_heads;
  int g = h / G;
  int64_t page = p->k_table[(int64_t)b * p->table_stride + j / p->page_size];
  int64_t off = key_offset(page, g, j % p->page_size, p->k_page_stride, p->k_head_stride,
                           p->k_tok_stride);
  int64_t qoff = (t * p->num_qo_heads + h) * (int64_t)p->head_dim_qk;
  double dot = 0.0;
  for (int d = 0; d < p->head_dim_qk; ++d)
    dot += load_elem(p->q, p->q_dtype, qoff + d) * load_elem(p->k, p->k_dtype, off + d);
  return p->scale * p->k_scale * dot;
}

static void value_row(const orc_problem* p, int b, int h, int64_t j, double* vrow) {
  int G = p->num_qo_heads / p->num_kv_heads;
  int g = h / G;
  int64_t page = p->v_table[(int64_t)b * p->table_stride + j / p->page_size];
  int64_t off = key_offset(page, g, j % p->page_size, p->v_page_stride, p->v_head_stride,
                           p->v_tok_stride);
  for (int d = 0; d < p->head_dim_v; ++d) vrow[d] = load_elem(p->v, p->v_dtype, off + d);
}

/* Fold a sink logit into a finished row: its weight joins the denominator. */
static void apply_sink(double* out, int dv, double* lse, double sigma) {
  double a = *lse, hi = a > sigma ? a : sigma;
  double lse2 = hi + log(exp(a - hi) + exp(sigma - hi));  /* a = -inf gives sigma */
  double f = exp(a - lse2);
  for (int d = 0; d < dv; ++d) out[d] *= f;
  *lse = lse2;
}

/* softmax-weighted mean over keys [j0, j1) for (row t, head h).
 * Writes the normalized output (times v_scale) and the natural-log LSE;
 * an empty range gives zeros and -inf. */
static void attend_range(const orc_problem* p, int b, int64_t t, int h, int64_t j0, int64_t j1,
                         double* out, double* lse, double* s, double* vrow) {
  int Dv = p->head_dim_v;
  for (int d = 0; d < Dv; ++d) out[d] = 0.0;
  if (j1 <= j0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t j = j0; j < j1; ++j) {
    s[j - j0] = logit(p, b, t, h, j);
    if (s[j - j0] > m) m = s[j - j0];
  }
  double l = 0.0;
  for (int64_t j = j0; j < j1; ++j) {
    double w = exp(s[j - j0] - m);
    l += w;
    value_row(p, b, h, j, vrow);
    for (int d = 0; d < Dv; ++d) out[d] += w * vrow[d];
  }
  for (int d = 0; d < Dv; ++d) out[d] = p->v_scale * out[d] / l;
  *lse = m + log(l);
}

static int64_t max_kv(const orc_problem* p) {
  int64_t mx = 0;
  for (int b = 0; b < p->batch; ++b)
    if (p->seq_lens[b] > mx) mx = p->seq_lens[b];
  return mx;
}

/*
 * Attention for n (row, head) pairs: pairs[2k] = global query row t,
 * pairs[2k+1] = query head h.  out is [n, head_dim_v], lse is [n] (may be NULL).
 * Returns 0, or -1 on a malformed pair.
 */
int orc_attention(const orc_problem* p, const int64_t* pairs, int64_t n, double* out,
                  double* lse) {
  int64_t cap = max_kv(p) + 1;
  double* s = (double*)malloc(sizeof(double) * (size_t)cap);
  double* vrow = (double*)malloc(sizeof(double) * (size_t)(p->head_dim_v + 1));
  if (!s || !vrow) {
    free(s);
    free(vrow);
    return -2;
  }
  int rc = 0;
  for (int64_t k = 0; k < n; ++k) {
    int64_t t = pairs[2 * k];
    int h = (int)pairs[2 * k + 1];
    int b = find_request(p, t);
    if (b < 0 || h < 0 || h >= p->num_qo_heads) {
      rc = -1;
      break;
    }
    double l_out;
    attend_range(p, b, t, h, 0, visible_keys(p, b, t), out + k * p->head_dim_v, &l_out, s, vrow);
    if (p->sinks) apply_sink(out + k * p->head_dim_v, p->head_dim_v, &l_out, p->sinks[h]);
    if (lse) lse[k] = l_out;
  }
  free(s);
  free(vrow);
  return rc;
}

/*
 * Split mode: the visible range [0, c) of each pair is cut at page-aligned
 * boundaries into num_splits partitions of ceil(ceil(L_b / P) / num_splits)
 * pages each (trailing partitions may be empty).  o_part is
 * [num_splits, n, head_dim_v] (each partition normalized on its own, times
 * v_scale), lse_part is [num_splits, n].
 */
int orc_attention_split(const orc_problem* p, int num_splits, const int64_t* pairs, int64_t n,
                        double* o_part, double* lse_part) {
  if (num_splits < 1) return -1;
  int64_t cap = max_kv(p) + 1;
  double* s = (double*)malloc(sizeof(double) * (size_t)cap);
  double* vrow = (double*)malloc(sizeof(double) * (size_t)(p->head_dim_v + 1));
  if (!s || !vrow) {
    free(s);
    free(vrow);
    return -2;
  }
  int rc = 0;
  for (int64_t k = 0; k < n && rc == 0; ++k) {
    int64_t t = pairs[2 * k];
    int h = (int)pairs[2 * k + 1];
    int b = find_request(p, t);
    if (b < 0 || h < 0 || h >= p->num_qo_heads) {
      rc = -1;
      break;
    }
    int64_t c = visible_keys(p, b, t);
    int64_t pages = (p->seq_lens[b] + p->page_size - 1) / p->page_size;
    int64_t pps = (pages + num_splits - 1) / num_splits;
    for (int sp = 0; sp < num_splits; ++sp) {
      int64_t j0 = (int64_t)sp * pps * p->page_size;
      int64_t j1 = (int64_t)(sp + 1) * pps * p->page_size;
      if (j1 > c) j1 = c;
      attend_range(p, b, t, h, j0, j1, o_part + ((int64_t)sp * n + k) * p->head_dim_v,
                   lse_part + (int64_t)sp * n + k, s, vrow);
    }
  }
  free(s);
  free(vrow);
  return rc;
}

/* Log-sum-exp merge of num_splits partial results (layouts as above); row k's
 * sink logit row_sinks[k] is applied once to the merged row when row_sinks is
 * not NULL. */
int orc_merge(int num_splits, int64_t n, int head_dim_v, const double* o_part,
              const double* lse_part, double* out, double* lse, const double* row_sinks) {
  for (int64_t k = 0; k < n; ++k) {
    double mx = -INFINITY;
    for (int sp = 0; sp < num_splits; ++sp)
      if (lse_part[(int64_t)sp * n + k] > mx) mx = lse_part[(int64_t)sp * n + k];
    double* o = out + k * head_dim_v;
    for (int d = 0; d < head_dim_v; ++d) o[d] = 0.0;
    if (mx == -INFINITY) {
      double l_empty = -INFINITY;
      if (row_sinks) apply_sink(o, head_dim_v, &l_empty, row_sinks[k]);
      if (lse) lse[k] = l_empty;
      continue;
    }
    double wsum = 0.0;
    for (int sp = 0; sp < num_splits; ++sp) {
      double ls = lse_part[(int64_t)sp * n + k];
      double w = (ls == -INFINITY) ? 0.0 : exp(ls - mx);
      wsum += w;
      const double* os = o_part + ((int64_t)sp * n + k) * head_dim_v;
      for (int d = 0; d < head_dim_v; ++d) o[d] += w * os[d];
    }
    for (int d = 0; d < head_dim_v; ++d) o[d] /= wsum;
    double l_row = mx + log(wsum);
    if (row_sinks) apply_sink(o, head_dim_v, &l_row, row_sinks[k]);
    if (lse) lse[k] = l_row;
  }
  return 0;
}

/*
 * pkv.h -- C ABI of libpkv.so, an MI355X (gfx950) paged-KV attention library.
 *
 * The library runs batched attention over a paged KV cache: every query row
 * reads its request's keys and values through a block table of fixed-size,
 * arbitrarily placed pages, runs an online softmax, and (when the planner
 * splits the KV range) writes per-partition partial outputs that a separate
 * log-sum-exp reducer merges.
 *
 * The call contract follows the paged decode and context ABIs described on
 * the flashinfer.cake_fmha API page: query, paged K/V cache (HND or NHD),
 * block_tables, seq_lens, max_kv_len, the softmax scale and optional scalar
 * FP8 scales go in; a caller-owned output comes out, enqueued on the caller's
 * stream.  The MLA form (one latent KV head whose first 512 channels are V)
 * follows the PR #4557 page's MLA decode description.
 *
 * Ownership and threading
 *   - Every pointer in pkv_args is a DEVICE pointer owned by the caller, except
 *     the pkv_args struct itself (host memory, read during the call only).
 *   - The library allocates nothing on the device and never synchronizes the
 *     host with the device.  Work is enqueued on `stream` (a hipStream_t passed
 *     as void*; NULL = the null stream) and may still be running on return.
 *   - Split-KV partials live in a caller-owned workspace whose size comes from
 *     pkv_workspace_bytes() for the same arguments.
 *   - Nothing is cached between calls: device values (seq_lens, tables,
 *     q_indptr) are read by the kernels on every call.
 *   - Entry points are thread-safe; pkv_last_error() is per host thread.
 *
 * Errors
 *   Host-checkable argument problems return PKV_ERR_INVALID_ARG before anything
 *   is enqueued.  Shapes or dtypes with no kernel return PKV_ERR_UNSUPPORTED
 *   (fail closed).  Device values are never trusted for addressing: a request
 *   uses L = min(seq_lens[b], span) keys, where span is the table capacity
 *   max_pages_per_seq * page_size or, for a Split-KV plan sized from max_kv_len
 *   (num_splits partitions of pages_per_split pages, pkv_plan_info), the
 *   num_splits * pages_per_split * page_size keys those partitions cover when
 *   that is smaller; page indices are clamped to [0, num_pages) when
 *   num_pages > 0.  A request with seq_lens[b] < its query rows, seq_lens[b] >
 *   max_pages_per_seq * page_size, seq_lens[b] > max_kv_len, or a referenced
 *   table entry outside [0, num_pages) sets the optional device error word
 *   (bit flags PKV_DEVERR_*) -- the PR #4557 page's review insists that the
 *   lengths a plan was made for stay tied to the call, so a stale host bound
 *   is reported rather than silently truncating; rows with no visible key
 *   produce zeros and lse = -inf.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 6

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* host-checkable argument violation */
  PKV_ERR_UNSUPPORTED = 2, /* valid arguments, but no kernel for them (fail closed) */
  PKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than pkv_workspace_bytes() */
  PKV_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} pkv_status;

typedef enum pkv_dtype {
  PKV_DTYPE_F32 = 0,
  PKV_DTYPE_BF16 = 1,
  PKV_DTYPE_FP8_E4M3 = 2 /* OCP e4m3 ("fn": max 448, no inf, 0x7F/0xFF NaN); KV only */
} pkv_dtype;

typedef enum pkv_layout {
  PKV_LAYOUT_HND = 0, /* pool [num_pages, Hkv, page_size, D]: one contiguous block per (page, head) */
  PKV_LAYOUT_NHD = 1  /* pool [num_pages, page_size, Hkv, D] */
} pkv_layout;

/* device error word bits (OR-ed; 0 = every request was well formed) */
#define PKV_DEVERR_SEQ_LT_QLEN 0x1    /* seq_lens[b] smaller than the request's query rows */
#define PKV_DEVERR_SEQ_GT_TABLE 0x2   /* seq_lens[b] > max_pages_per_seq * page_size (clamped) */
#define PKV_DEVERR_PAGE_RANGE 0x4     /* a referenced page index outside [0, num_pages) (clamped) */
#define PKV_DEVERR_QINDPTR 0x8        /* q_indptr not monotone, or rows exceed max_q_len / total_q */
#define PKV_DEVERR_POS_RANGE 0x10     /* pkv_append: a row's position is past the rotary table */
#define PKV_DEVERR_QSCALE_ROWS 0x20   /* pkv_append: a request has more new rows than q_scale_stride */
#define PKV_DEVERR_SEQ_GT_MAXLEN 0x40 /* seq_lens[b] > max_kv_len, the host bound the plan was sized from:
                                         keys past the planned span are not read (clamped) */

/*
 * Arguments of one attention call.  Strides are in ELEMENTS of the tensor's
 * dtype; the innermost (head-dim) stride is always 1.
 *
 * Query / output rows.  Decode (pkv_decode): request b owns rows
 * b*q_len .. b*q_len+q_len-1 (q_len = 1 is plain decode, q_len > 1 are
 * speculative rows).  Context (pkv_context): request b owns rows
 * q_indptr[b] .. q_indptr[b+1]-1.  Row t, head h lives at
 * q + t*q_stride_tok + h*q_stride_head (likewise out / o_stride_*).
 *
 * Keys.  seq_lens[b] is the request's total KV length INCLUDING its own query
 * rows.  With causal != 0, row i (0-based within the request, n rows) sees keys
 * 0 .. seq_lens[b] - n + i (inclusive); otherwise all seq_lens[b] keys.  Key j
 * of request b is token j % page_size of page block_tables[b*table_stride + j/page_size];
 * its K row for KV head g starts at
 *     k_pages + page*k_stride_page + g*k_stride_head + (j % page_size)*k_stride_tok.
 * Query head h uses KV head h / (num_qo_heads / num_kv_heads).
 *
 * Scores and output:
 *     s_j = scale * k_scale * <q, k_j>,   out = v_scale * sum_j softmax(s)_j v_j
 * k_scale / v_scale are 1 except for FP8 KV (stored value = x / scale).  When
 * k_scale_dev / v_scale_dev are non-NULL they point to device float scalars
 * that replace k_scale / v_scale.  lse_out (optional, fp32 [total_q, Hq] with
 * row stride num_qo_heads) receives the natural-log log-sum-exp of the scores.
 */
typedef struct pkv_args {
  int32_t batch;             /* B >= 0; B == 0 is a no-op */
  int32_t q_len;             /* decode: query rows per request (>= 1); context: ignored */
  int32_t num_qo_heads;      /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;      /* Hkv >= 1 */
  int32_t head_dim_qk;       /* D_qk, multiple of 8 */
  int32_t head_dim_v;        /* D_v, multiple of 8, <= head_dim_qk when v_shares_k */
  int32_t page_size;         /* P >= 1 */
  int32_t max_pages_per_seq; /* readable width of each block-table row */
  int32_t max_kv_len;        /* host upper bound on seq_lens (sizes the Split-KV plan); a device
                                length above it is flagged (PKV_DEVERR_SEQ_GT_MAXLEN) and cut
                                to the planned span */
  int32_t max_q_len;         /* context: host upper bound on rows per request */
  int32_t total_q;           /* context: rows of q / out (= q_indptr[B]); decode: ignored */
  int32_t num_pages;         /* pool size in pages for clamping, 0 = unchecked */
  int32_t q_dtype;           /* pkv_dtype: F32 or BF16 */
  int32_t kv_dtype;          /* pkv_dtype: F32, BF16 or FP8_E4M3 */
  int32_t o_dtype;           /* pkv_dtype: F32 or BF16 */
  int32_t layout;            /* pkv_layout (only used to validate strides) */
  int32_t causal;            /* 1: inclusive causal bound for multi-row requests */
  int32_t num_splits;        /* Split-KV partitions per (request, KV head); 0 = planner;
                                -1 = balanced decode schedule (GQA decode families only) */
  int32_t v_shares_k;        /* 1: V is the first head_dim_v channels of the K rows (MLA) */
  int32_t kernel_hint;       /* 0: planner picks; else a pkv_plan_info.kernel id to force
                                (PKV_ERR_UNSUPPORTED when that family cannot run the shape) */

  const void* q;
  const void* k_pages;
  const void* v_pages;       /* ignored when v_shares_k */
  const int32_t* block_tables;
  const int32_t* seq_lens;   /* [B] */
  const int32_t* q_indptr;   /* context: [B + 1]; decode: ignored */
  void* out;
  float* lse_out;            /* optional */
  int32_t* err_word;         /* optional device word, OR-ed with PKV_DEVERR_* bits */
  const float* k_scale_dev;  /* optional */
  const float* v_scale_dev;  /* optional */
  /* Optional split counters for the balanced decode schedule (num_splits == -1,
     or chosen by the planner): int32 [pkv_plan_info.counter_words], device
     memory that must be all zero before its first use (e.g. allocated zeroed
     once) and that every completed call leaves all zero again.  With it, the
     last workgroup to finish a (request, KV head) merges that unit's partial
     rows inside the attention kernel (the PR #4557 page: split counters in
     caller-owned memory that reset themselves); NULL selects the separate
     reducer kernel.  Calls that share one counter buffer must not overlap in
     time (same stream, or otherwise ordered).  Ignored by every other plan. */
  int32_t* merge_counters;
  /* Optional attention sinks: fp32 [num_qo_heads] device array, one logit per
     query head in the units of the scaled scores (scale * k_scale * q.k).  Its
     weight joins each row's softmax denominator and carries no value:
     lse = ln(sum_j e^{s_j} + e^{sink}) and the output shrinks by the same
     factor; a row with no visible key reports lse = sink.  The pages list
     `sinks` among the decode arguments (PR #4557 page, MLA dispatcher excerpt)
     without defining them: this is the reading taken.  NULL: no sink. */
  const float* sinks;
  /* Optional separate V page table [B, table_stride] (flashinfer.cake_fmha API
     page: a context profile with separate K/V page tables): value j of request
     b is read from page v_block_tables[b][j / P].  NULL: V shares block_tables.
     Served by every D = 128 family (each keeps a second page list beside
     the K list, also on the balanced schedule) and the generic kernel; a
     kernel_hint of an MLA family returns PKV_ERR_UNSUPPORTED (its V rows are
     the K rows).  Page indices are clamped and flagged like K's. */
  const int32_t* v_block_tables;

  int64_t q_stride_tok, q_stride_head;
  int64_t o_stride_tok, o_stride_head;
  int64_t k_stride_page, k_stride_head, k_stride_tok;
  int64_t v_stride_page, v_stride_head, v_stride_tok;
  int64_t table_stride;

  float scale;
  float k_scale;
  float v_scale;
  float reserved1;
} pkv_args;

/* Planner result (host only, no device access). */
typedef struct pkv_plan_info {
  int32_t kernel;          /* internal kernel family id (stable within one ABI version) */
  int32_t num_splits;      /* partitions per (request, KV head) */
  int32_t pages_per_split; /* page-aligned partition length, in pages */
  int32_t grid_x, grid_y, grid_z;
  int32_t block_threads;
  int32_t schedule;        /* 0: per-unit partitions, grid (num_splits, Hkv x row blocks, B);
                              1: balanced decode schedule, grid_x workgroups own equal page
                                 ranges of all requests; num_splits then counts partial slots */
  int32_t counter_words;   /* schedule 1: int32 words merge_counters must hold (B x Hkv); else 0 */
  int32_t fused_merge;     /* 1: the reducer runs inside the attention kernel (merge_counters given) */
  size_t workspace_bytes;  /* 0 when num_splits == 1 */
} pkv_plan_info;

/* ABI version of the loaded library (PKV_ABI_VERSION of the headers it was built from). */
int pkv_abi_version(void);

/* Message for the last non-OK status returned on this host thread ("" if none). */
const char* pkv_last_error(void);

/*
 * Host-only planning for pkv_decode (is_context = 0) or pkv_context (1):
 * validates the host-visible arguments, picks the kernel, the Split-KV
 * partition count sized to the device's compute units (num_cus <= 0 = 256) and
 * the workspace size.  Pointers are not dereferenced.
 */
pkv_status pkv_plan(const pkv_args* args, int is_context, int num_cus, pkv_plan_info* info);

/*
 * Workspace bytes pkv_decode / pkv_context need for these arguments (0 if
 * unsplit).  The caller owns the workspace and sizes it with this query, and
 * no call path allocates device memory: the caller-owned-workspace item of
 * the DeepSeek-V4 hardening summary (#5591) on the PR #4557 page.  The plan
 * behind the size is made for the compute-unit count of the CURRENT device
 * (hipGetDevice at the time of the call), the same count pkv_decode and
 * pkv_context plan with, so query and call on the same device.  pkv_plan's
 * num_cus argument serves host-side inspection of other counts.
 */
pkv_status pkv_workspace_bytes(const pkv_args* args, int is_context, size_t* bytes);

/*
 * Paged decode: B requests with q_len uniform query rows each (speculative rows
 * are causal within the draft when args->causal).  The Split-KV partials go
 * into `workspace` (device, >= pkv_workspace_bytes bytes, 256-byte aligned) and
 * are merged by the log-sum-exp reducer in the same call.
 */
pkv_status pkv_decode(const pkv_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* Paged causal context (prefill): variable rows per request through args->q_indptr. */
pkv_status pkv_context(const pkv_args* args, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_decode without a workspace argument, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same plan and kernels as pkv_decode; the Split-KV partials
 * live in a static device array of PKV_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends (its device address is
 * looked up once per device).  The call allocates nothing and frees nothing.
 * A call whose plan needs more scratch returns PKV_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (no call relies on it starting at zero):
 * calls that may overlap on one GPU (different streams, or several host
 * threads) race and must not be issued.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
pkv_status pkv_decode_noalloc(const pkv_args* args, void* stream);

/*
 * The log-sum-exp reducer on its own (Split-KV merge, PR #4557 page: split
 * partitions merged by a separate reducer kernel).
 *   o_part   fp32 [num_splits, num_rows, head_dim_v], each partition normalized
 *   lse_part fp32 [num_splits, num_rows] natural log, -inf = empty partition
 * Row r is (query row r / num_qo_heads, head r % num_qo_heads); the merged
 * row goes to out + (r / Hq)*o_stride_tok + (r % Hq)*o_stride_head in o_dtype
 * and its log-sum-exp to lse_out[r] when lse_out is non-NULL.  Rows whose
 * partitions are all empty produce zeros and -inf.
 */
pkv_status pkv_lse_merge(int32_t num_splits, int32_t num_rows, int32_t num_qo_heads,
                         int32_t head_dim_v, const float* o_part, const float* lse_part,
                         void* out, int32_t o_dtype, int64_t o_stride_tok, int64_t o_stride_head,
                         float* lse_out, void* stream);

/* ---------------------------------------------------------------- paged KV append (the producer) */

/*
 * Fused QK RMSNorm + NeoX rotary embedding + paged K/V append, one launch
 * (PR #5952 page, summary; the PR #5956 body quoted there, section "Contract").
 * Packed row r of request b (rows q_indptr[b] .. q_indptr[b+1] of qkv) sits at
 * position pos = r + seq_lens[b] - q_indptr[b+1] (seq_lens = total length
 * after the append) and holds Hq query heads, Hkv key heads and Hkv value
 * heads of 128 channels each, in that order.
 *   - query and key heads: the norm policy (0 none; 1 rotary then RMSNorm;
 *     2 RMSNorm then rotary), RMSNorm y = x / sqrt(mean(x^2) + eps) * w in fp32
 *     with w = q_weight or k_weight, and the NeoX rotary embedding with row pos
 *     of cos_sin = (cos_0..63, sin_0..63): channel i < 64 pairs with i + 64,
 *     y_i = x_i cos_i - x_{i+64} sin_i, y_{i+64} = x_{i+64} cos_i + x_i sin_i;
 *   - the query heads are written to out_q[r]: bf16 (round to nearest even)
 *     with q_quant = 0, else e4m3 codes (round to nearest even, saturated to
 *     +-448) of y / s with, for q_quant = 1, a scale of its own per (row,
 *     head) s = max(max_i |y_i|, 1e-6) / upper_max, written as fp32 to
 *     q_scale (q_scale_layout 0: [T, Hq], entry r * Hq + h; 1: [B, Hq,
 *     q_scale_stride], entry (b * Hq + h) * q_scale_stride + i for the i-th
 *     new row of request b -- the pages round the stride up to a multiple of
 *     128; entries of rows no request appends are left untouched), or, for
 *     q_quant = 2, of y * q_scale_inv with no scale written (PR #5956 body,
 *     "Contract": dynamic per-token/per-head or static query quantization);
 *   - key heads and the unchanged value heads are written to token pos % P of
 *     page block_tables[b][pos / P] of the caches: bf16, or e4m3 codes of
 *     x / k_scale and x / v_scale (round to nearest even, saturated to
 *     +-448).  The pages' caches are NHD [num_pages, P, Hkv, 128]; `layout`
 *     and the element strides also take the HND pools [num_pages, Hkv, P,
 *     128] the attention entry points read, so the row of slot s, KV head g
 *     of page pg starts at k_cache + pg*k_stride_page + g*k_stride_head +
 *     s*k_stride_tok (likewise V), with the same consistency rules as
 *     pkv_args' pools;
 *   - with clear_tail, tokens [(seq_lens[b] - 1) % P + 1, P) of every nonempty
 *     request's last page are zeroed in both caches (the caller owns the pages
 *     exclusively: a page shared with a longer request would lose rows).
 * A request whose rows do not fit (seq_lens[b] < rows, seq_lens[b] > max_pages_per_seq * P
 * or > max_pos, q_indptr not monotone or past num_tokens, more rows than
 * q_scale_stride in the dynamic [B, Hq, stride] layout) writes nothing and
 * sets PKV_DEVERR_* bits; a page index outside [0, num_pages) (num_pages > 0)
 * skips that row's cache write and sets PKV_DEVERR_PAGE_RANGE.  Device values
 * are never used for addressing unchecked.  Nothing is allocated, nothing
 * synchronizes the host; the work is enqueued on `stream` and can be captured
 * in a graph.  Returns PKV_ERR_INVALID_ARG / PKV_ERR_UNSUPPORTED for
 * host-checkable problems before anything is enqueued.
 */
typedef struct pkv_append_args {
  int32_t num_tokens;        /* T = q_indptr[B], rows of qkv and out_q (host value) */
  int32_t batch;             /* B >= 0; T = 0 with clear_tail = 0 (or B = 0) is a no-op */
  int32_t num_qo_heads;      /* Hq >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1 */
  int32_t head_dim;          /* 128 */
  int32_t page_size;         /* P >= 1 */
  int32_t max_pages_per_seq; /* readable width of each block-table row */
  int32_t max_pos;           /* rows of cos_sin */
  int32_t num_pages;         /* cache pages, for checking page indices (0 = unchecked) */
  int32_t norm_policy;       /* 0, 1 or 2 (above) */
  int32_t clear_tail;        /* 1: zero the tail of each nonempty request's last page */
  int32_t kv_dtype;          /* PKV_DTYPE_BF16 or PKV_DTYPE_FP8_E4M3 */
  float eps;                 /* RMSNorm epsilon (the pages use 1e-6), >= 0 */
  float k_scale;             /* e4m3 caches: stored = x / k_scale (finite, non-zero) */
  float v_scale;
  float reserved;
  const void* qkv;           /* bf16 [T, qkv_stride_tok], the first (Hq + 2 Hkv) * 128 used */
  int64_t qkv_stride_tok;    /* elements between rows, >= (Hq + 2 Hkv) * 128 */
  const float* cos_sin;      /* fp32 [max_pos, 128] */
  const void* q_weight;      /* bf16 [128]; read only when norm_policy != 0 */
  const void* k_weight;      /* bf16 [128] */
  const int32_t* q_indptr;   /* [B + 1] */
  const int32_t* seq_lens;   /* [B] */
  const int32_t* block_tables; /* [B, table_stride] */
  int64_t table_stride;      /* >= max_pages_per_seq */
  void* out_q;               /* [T, Hq, 128]: bf16 (q_quant 0) or e4m3 codes */
  void* k_cache;             /* [num_pages, P, Hkv, 128] (NHD) or [num_pages, Hkv, P, 128] (HND), bf16 or e4m3 */
  void* v_cache;
  int32_t* err_word;         /* optional device word, OR-ed with PKV_DEVERR_* bits */
  int32_t q_quant;           /* query output: 0 bf16; 1 e4m3, dynamic scale; 2 e4m3, static scale */
  float upper_max;           /* q_quant 1: finite, in (0, 448] */
  float q_scale_inv;         /* q_quant 2: finite, non-zero */
  int32_t q_scale_layout;    /* q_quant 1: 0 [T, Hq] or 1 [B, Hq, q_scale_stride] */
  int64_t q_scale_stride;    /* q_scale_layout 1: entries per (request, head), >= 1 */
  float* q_scale;            /* q_quant 1: fp32 scales (layout above), 4-byte aligned */
  int32_t layout;            /* pkv_layout of both caches (validates the strides) */
  int32_t reserved2;
  int64_t k_stride_page, k_stride_head, k_stride_tok; /* K cache strides in elements of kv_dtype */
  int64_t v_stride_page, v_stride_head, v_stride_tok; /* V cache strides */
} pkv_append_args;

pkv_status pkv_append(const pkv_append_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

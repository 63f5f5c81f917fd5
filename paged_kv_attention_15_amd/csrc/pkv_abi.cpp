// pkv_abi.cpp -- the extern "C" boundary of libpkv.so: validation, planning, launches.
//
// The call contract (query, paged K/V, block tables, seq_lens, max_kv_len,
// scale and scalar FP8 scales in, caller-owned output out, on the caller's
// stream) follows the flashinfer.cake_fmha API page; unsupported combinations
// fail closed with PKV_ERR_UNSUPPORTED as that page's optimized routes do.
// Nothing here reads device memory, allocates, synchronizes, or caches state
// keyed on pointers (PR #4557 page: host metadata must stay bound to the
// tensors of the current call).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/pkv.h"
#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

int elem_bytes(int32_t dt) {
  switch (dt) {
    case PKV_DTYPE_F32: return 4;
    case PKV_DTYPE_BF16: return 2;
    case PKV_DTYPE_FP8_E4M3: return 1;
  }
  return 0;
}

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int64_t x) {
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

constexpr int kMaxSplits = 256;
constexpr int kMaxPagesPerSplit = 4096;  // bounds the LDS page list of the MFMA kernels

// Strides (elements) of a paged pool [pages, Hkv, P, D] (HND) or [pages, P,
// Hkv, D] (NHD), innermost contiguous: rows of one page never overlap and
// every page holds all of its rows.
pkv_status check_pool_strides(int32_t layout, int64_t H, int64_t P, int64_t D, int64_t sp, int64_t sh, int64_t st,
                              const char* name) {
  if (sp <= 0 || sh < 0 || st <= 0) return fail(PKV_ERR_INVALID_ARG, "%s strides must be positive", name);
  if (layout == PKV_LAYOUT_HND) {
    if (st < D || (H > 1 && sh < P * st) || sp < H * std::max<int64_t>(sh, P * st))
      return fail(PKV_ERR_INVALID_ARG, "%s strides do not describe an HND [pages, Hkv, P, D] pool", name);
  } else {
    if ((H > 1 && sh < D) || st < H * std::max<int64_t>(sh, D) || sp < P * st)
      return fail(PKV_ERR_INVALID_ARG, "%s strides do not describe an NHD [pages, P, Hkv, D] pool", name);
  }
  return PKV_OK;
}

// Host-visible argument checks shared by plan / decode / context.
pkv_status validate(const pkv_args* a, bool is_context) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  if ((reinterpret_cast<uintptr_t>(a->merge_counters) & 3u) != 0)
    return fail(PKV_ERR_INVALID_ARG, "merge_counters must be 4-byte aligned");
  if (a->v_block_tables && a->v_shares_k)
    return fail(PKV_ERR_INVALID_ARG, "v_block_tables with v_shares_k: V rows are the K rows");
  if ((reinterpret_cast<uintptr_t>(a->sinks) | reinterpret_cast<uintptr_t>(a->v_block_tables)) & 3u)
    return fail(PKV_ERR_INVALID_ARG, "sinks and v_block_tables must be 4-byte aligned");
  if (a->batch < 0) return fail(PKV_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", a->batch);
  if (a->num_kv_heads < 1 || a->num_qo_heads < 1 || a->num_qo_heads % a->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_qo_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_qo_heads, a->num_kv_heads);
  if (a->head_dim_qk < 8 || a->head_dim_qk % 8 != 0 || a->head_dim_v < 8 || a->head_dim_v % 8 != 0)
    return fail(PKV_ERR_INVALID_ARG, "head dims must be positive multiples of 8 (qk %d, v %d)", a->head_dim_qk,
                a->head_dim_v);
  if (a->v_shares_k && a->head_dim_v > a->head_dim_qk)
    return fail(PKV_ERR_INVALID_ARG, "v_shares_k needs head_dim_v <= head_dim_qk");
  if (a->page_size < 1) return fail(PKV_ERR_INVALID_ARG, "page_size must be >= 1 (got %d)", a->page_size);
  if (a->max_pages_per_seq < 0) return fail(PKV_ERR_INVALID_ARG, "max_pages_per_seq must be >= 0");
  if (a->max_kv_len < 0) return fail(PKV_ERR_INVALID_ARG, "max_kv_len must be >= 0");
  if ((int64_t)a->max_kv_len > (int64_t)a->max_pages_per_seq * a->page_size)
    return fail(PKV_ERR_INVALID_ARG, "max_kv_len %d exceeds the table capacity %lld", a->max_kv_len,
                (long long)a->max_pages_per_seq * a->page_size);
  if ((int64_t)a->max_pages_per_seq * a->page_size > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "max_pages_per_seq * page_size exceeds 2^31 - 1 keys");
  if (a->num_pages < 0) return fail(PKV_ERR_INVALID_ARG, "num_pages must be >= 0");
  if (a->q_dtype != PKV_DTYPE_F32 && a->q_dtype != PKV_DTYPE_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "q_dtype %d not supported (F32 or BF16)", a->q_dtype);
  if (a->o_dtype != PKV_DTYPE_F32 && a->o_dtype != PKV_DTYPE_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "o_dtype %d not supported (F32 or BF16)", a->o_dtype);
  if (elem_bytes(a->kv_dtype) == 0) return fail(PKV_ERR_UNSUPPORTED, "kv_dtype %d not supported", a->kv_dtype);
  if (a->layout != PKV_LAYOUT_HND && a->layout != PKV_LAYOUT_NHD)
    return fail(PKV_ERR_INVALID_ARG, "layout %d unknown", a->layout);
  if (!(a->scale > 0.f) || !(a->k_scale > 0.f) || !(a->v_scale > 0.f))
    return fail(PKV_ERR_INVALID_ARG, "scale, k_scale and v_scale must be positive and finite");
  if (a->num_splits < -1 || a->num_splits > kMaxSplits)
    return fail(PKV_ERR_INVALID_ARG, "num_splits must be -1 (balanced schedule), 0 (planner) or in [1, %d]",
                kMaxSplits);
  if (is_context) {
    if (a->max_q_len < 0 || a->total_q < 0) return fail(PKV_ERR_INVALID_ARG, "max_q_len / total_q must be >= 0");
  } else {
    if (a->q_len < 1) return fail(PKV_ERR_INVALID_ARG, "q_len must be >= 1 for decode (got %d)", a->q_len);
    if ((int64_t)a->q_len > (int64_t)a->max_pages_per_seq * a->page_size && a->batch > 0)
      return fail(PKV_ERR_INVALID_ARG, "q_len exceeds the table capacity");
  }
  // query rows x heads index the reducer's grid and its 32-bit row arithmetic
  const int64_t q_rows = (is_context ? (int64_t)a->total_q : (int64_t)a->batch * a->q_len) * a->num_qo_heads;
  if (q_rows > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "query rows x heads (%lld) exceed 2^31 - 1", (long long)q_rows);
  // layout consistency of the strides (innermost dimension contiguous)
  const int64_t D_qk = a->head_dim_qk, D_v = a->head_dim_v;
  pkv_status st = check_pool_strides(a->layout, a->num_kv_heads, a->page_size, D_qk, a->k_stride_page,
                                     a->k_stride_head, a->k_stride_tok, "k");
  if (st != PKV_OK) return st;
  if (!a->v_shares_k) {
    st = check_pool_strides(a->layout, a->num_kv_heads, a->page_size, D_v, a->v_stride_page, a->v_stride_head,
                            a->v_stride_tok, "v");
    if (st != PKV_OK) return st;
  }
  if (a->table_stride < a->max_pages_per_seq)
    return fail(PKV_ERR_INVALID_ARG, "table_stride %lld < max_pages_per_seq %d", (long long)a->table_stride,
                a->max_pages_per_seq);
  if (a->q_stride_head < D_qk || a->q_stride_tok < D_qk)
    return fail(PKV_ERR_INVALID_ARG, "q strides too small for head_dim_qk");
  if (a->o_stride_head < D_v || a->o_stride_tok < D_v)
    return fail(PKV_ERR_INVALID_ARG, "out strides too small for head_dim_v");
  if (a->batch == 0) return PKV_OK;
  if (!a->q || !a->k_pages || (!a->v_shares_k && !a->v_pages) || !a->block_tables || !a->seq_lens || !a->out)
    return fail(PKV_ERR_INVALID_ARG, "q, k_pages, v_pages, block_tables, seq_lens and out are required");
  if (is_context && !a->q_indptr) return fail(PKV_ERR_INVALID_ARG, "q_indptr is required for context");
  return PKV_OK;
}

// Can the MFMA families run these arguments at all (dtypes, power-of-two pages,
// 16-byte aligned rows)?  Anything they cannot prove safe goes to the generic
// kernel (fail-closed routing).
bool mfma_eligible(const pkv_args* a) {
  const bool mfma_kv = a->kv_dtype == PKV_DTYPE_BF16 || a->kv_dtype == PKV_DTYPE_FP8_E4M3;
  const int eb = elem_bytes(a->kv_dtype);
  if (a->q_dtype != PKV_DTYPE_BF16 || !mfma_kv || !is_pow2(a->page_size)) return false;
  auto al = [&](int64_t stride_elems, int bytes) { return (stride_elems * bytes) % 16 == 0; };
  if (!aligned16(a->q) || !aligned16(a->k_pages) || !aligned16(a->out)) return false;
  if (!a->v_shares_k && !aligned16(a->v_pages)) return false;
  if (!al(a->q_stride_tok, 2) || !al(a->q_stride_head, 2)) return false;
  const int ob = elem_bytes(a->o_dtype);
  if ((a->o_stride_tok * ob) % 8 != 0 || (a->o_stride_head * ob) % 8 != 0) return false;
  if (!al(a->k_stride_page, eb) || !al(a->k_stride_head, eb) || !al(a->k_stride_tok, eb)) return false;
  if (!a->v_shares_k && (!al(a->v_stride_page, eb) || !al(a->v_stride_head, eb) || !al(a->v_stride_tok, eb)))
    return false;
  return true;
}

// Does kernel family k cover these arguments?
bool kernel_supports(int32_t k, const pkv_args* a, bool is_context) {
  if (k == pkv::KERNEL_GENERIC) return a->head_dim_qk <= 1024 && a->head_dim_v <= 512;
  if (k <= pkv::KERNEL_GENERIC || k >= pkv::KERNEL_COUNT || !mfma_eligible(a)) return false;
  // separate V tables: every D = 128 family keeps a second page list; the MLA
  // kernels read V from the K rows and take none
  pkv::MfmaShape ring;
  const bool ring_family = pkv::dma_shape(k, &ring);
  if (a->v_block_tables && (k == pkv::KERNEL_MLA_BF16 || k == pkv::KERNEL_MLA_FP8 || k == pkv::KERNEL_MLA32_BF16 ||
                            k == pkv::KERNEL_DMA_MLA_BF16 || k == pkv::KERNEL_DMA_MLA_FP8))
    return false;
  // the direct-to-LDS ring loaders form a page's address as a 64-bit base
  // plus a 32-bit product and offset: pages of 4 GiB or more go elsewhere
  const int64_t eb = elem_bytes(a->kv_dtype);
  if (ring_family &&
      (a->k_stride_page * eb > (int64_t)UINT32_MAX || (!a->v_shares_k && a->v_stride_page * eb > (int64_t)UINT32_MAX)))
    return false;
  const bool fp8 = a->kv_dtype == PKV_DTYPE_FP8_E4M3;
  const int G = a->num_qo_heads / a->num_kv_heads;
  const bool d128 = a->head_dim_qk == 128 && a->head_dim_v == 128 && !a->v_shares_k;
  const bool mla = a->head_dim_qk == 576 && a->head_dim_v == 512 && a->v_shares_k;
  switch (k) {
    case pkv::KERNEL_GQA_BF16: return d128 && !fp8 && !is_context && (int64_t)a->q_len * G <= 16;
    case pkv::KERNEL_GQA_FP8:
    case pkv::KERNEL_DMA_GQA_FP8_N2: return d128 && fp8 && !is_context && (int64_t)a->q_len * G <= 16;
    case pkv::KERNEL_WIDE_BF16: return d128 && !fp8;
    case pkv::KERNEL_WIDE_FP8: return d128 && fp8;
    case pkv::KERNEL_MLA_BF16: return mla && !fp8;
    case pkv::KERNEL_MLA_FP8: return mla && fp8;
    case pkv::KERNEL_DMA_WIDE_BF16: return d128 && !fp8;
    case pkv::KERNEL_DMA_WIDE_FP8: return d128 && fp8;
    case pkv::KERNEL_DMA_MLA_BF16: return mla && !fp8;
    case pkv::KERNEL_DMA_MLA_FP8: return mla && fp8;
    // the 32x32 context kernel loads four rows per wave-instruction from one page
    case pkv::KERNEL_M32_CTX_W8T128: return d128 && !fp8 && a->page_size >= 4;
    // 32-key blocks inside one page: pages of a multiple of 32 tokens
    case pkv::KERNEL_MLA32_BF16: return mla && !fp8 && a->page_size % 32 == 0;
  }
  return false;
}

// families that hold a partition's page list in registers (kM32MaxPages pages at most)
bool page_list_in_registers(int32_t k) { return k == pkv::KERNEL_M32_CTX_W8T128 || k == pkv::KERNEL_MLA32_BF16; }

bool is_m32(int32_t k) { return k == pkv::KERNEL_M32_CTX_W8T128; }
// the direct-to-LDS ring families (pkv_attn_dma.hip)
bool is_ring(int32_t k) {
  pkv::MfmaShape sh;
  return pkv::dma_shape(k, &sh);
}
bool is_mla32(int32_t k) { return k == pkv::KERNEL_MLA32_BF16; }

// families with a balanced decode schedule (rows of a KV head in one block)
bool is_gqa_family(int32_t k) {
  return k == pkv::KERNEL_GQA_BF16 || k == pkv::KERNEL_GQA_FP8 || k == pkv::KERNEL_DMA_GQA_FP8_N2;
}

bool kernel_shape(int32_t k, pkv::MfmaShape* s) {
  return pkv::mfma_shape(k, s) || pkv::dma_shape(k, s) || pkv::m32_shape(k, s) || pkv::mla32_shape(k, s);
}

// Balanced schedule: the fixed cost of starting a segment (page list and
// query loads, pipeline fill and drain), charged as placeholder pages of this
// request's page size.  48 KiB of K and V per segment start was the best of
// 0, 16, 32, 48 and 64 KiB on MI355X for the ragged e4m3 decode (16 requests,
// 8 KV heads, 64-token pages): 63.7, 61.5, 60.6, 59.3 and 59.6 us per call.
#ifndef PKV_SEG_COST_BYTES
#define PKV_SEG_COST_BYTES 49152
#endif
int32_t seg_cost_pages(const pkv_args* a) {
  const int eb = a->kv_dtype == PKV_DTYPE_FP8_E4M3 ? 1 : (a->kv_dtype == PKV_DTYPE_BF16 ? 2 : 4);
  const int64_t page_bytes =
      (int64_t)a->page_size * (a->head_dim_qk + (a->v_shares_k ? 0 : a->head_dim_v)) * eb;
  return (int32_t)std::min<int64_t>(64, (PKV_SEG_COST_BYTES + page_bytes / 2) / std::max<int64_t>(page_bytes, 1));
}

int32_t preferred_kernel(const pkv_args* a, bool is_context) {
  if (!mfma_eligible(a)) return pkv::KERNEL_GENERIC;
  const bool fp8 = a->kv_dtype == PKV_DTYPE_FP8_E4M3;
  const int G = a->num_qo_heads / a->num_kv_heads;
  // Measured on MI355X (bf16 GQA decode B32/L4096, e4m3 ragged decode B16, MLA
  // B512/L4096, causal context B4 q511/L2047): register-staged tiles win for
  // bf16 decode, the direct-to-LDS ring for e4m3 decode (two-wave groups, four
  // per CU) and MLA, the 32x32 MFMA family with two waves per SIMD for bf16
  // context, in the form with two 128-key stages (2-3 % faster than four 64-key
  // stages in five back-to-back pairs: half the workgroup barriers; 96-key
  // stages were 2-4 % slower; the variant with the next block's S^T interleaved
  // with the softmax measured within +-3 % of the 64-key form).
  if (a->head_dim_qk == 128 && a->head_dim_v == 128 && !a->v_shares_k) {
    const int64_t rows = is_context ? (int64_t)a->max_q_len * G : (int64_t)a->q_len * G;
    if (!is_context && rows <= 16) return fp8 ? pkv::KERNEL_DMA_GQA_FP8_N2 : pkv::KERNEL_GQA_BF16;
    if (is_context && !fp8) return pkv::KERNEL_M32_CTX_W8T128;
    return fp8 ? pkv::KERNEL_DMA_WIDE_FP8 : pkv::KERNEL_DMA_WIDE_BF16;
  }
  // MLA: bf16 latents on the 32x32 kernel with 32 heads per wave when the
  // pages hold whole 32-key blocks (B512 L4096: 686 us for one query row and
  // 1,199 us for two, against 746 / 1,381 us for the 16-head ring kernel)
  if (a->head_dim_qk == 576 && a->head_dim_v == 512 && a->v_shares_k) {
    if (!fp8 && a->page_size % 32 == 0) return pkv::KERNEL_MLA32_BF16;
    return fp8 ? pkv::KERNEL_DMA_MLA_FP8 : pkv::KERNEL_DMA_MLA_BF16;
  }
  return pkv::KERNEL_GENERIC;
}

// The preferred family, else (a direct-to-LDS ring family on pages it cannot
// address) its register-staged twin, else the generic kernel.
int32_t choose_kernel(const pkv_args* a, bool is_context) {
  const int32_t k = preferred_kernel(a, is_context);
  if (kernel_supports(k, a, is_context)) return k;
  int32_t twin = pkv::KERNEL_GENERIC;
  switch (k) {
    case pkv::KERNEL_DMA_GQA_FP8_N2: twin = pkv::KERNEL_GQA_FP8; break;
    case pkv::KERNEL_DMA_WIDE_FP8: twin = pkv::KERNEL_WIDE_FP8; break;
    case pkv::KERNEL_DMA_WIDE_BF16: twin = pkv::KERNEL_WIDE_BF16; break;
    case pkv::KERNEL_DMA_MLA_FP8: twin = pkv::KERNEL_MLA_FP8; break;
    case pkv::KERNEL_DMA_MLA_BF16: twin = pkv::KERNEL_MLA_BF16; break;
  }
  return kernel_supports(twin, a, is_context) ? twin : pkv::KERNEL_GENERIC;
}

pkv_status make_plan(const pkv_args* a, bool is_context, int num_cus, pkv_plan_info* info) {
  pkv_status st = validate(a, is_context);
  if (st != PKV_OK) return st;
  if (num_cus <= 0) num_cus = 256;
  std::memset(info, 0, sizeof *info);
  const int32_t kernel = a->kernel_hint ? a->kernel_hint : choose_kernel(a, is_context);
  if (!kernel_supports(kernel, a, is_context))
    return fail(PKV_ERR_UNSUPPORTED, a->kernel_hint ? "kernel_hint %d cannot run these arguments"
                                                    : "no kernel for these arguments (family %d)", kernel);
  info->kernel = kernel;
  const int G = a->num_qo_heads / a->num_kv_heads;
  const int64_t rows_per_kv = is_context ? (int64_t)a->max_q_len * G : (int64_t)a->q_len * G;
  const int64_t total_rows = is_context ? a->total_q : (int64_t)a->batch * a->q_len;
  const int64_t max_pages = (a->max_kv_len + a->page_size - 1) / a->page_size;

  int tile_tokens = 64, rows_per_block = 1, threads = 64;
  int64_t units;  // independent (request, KV head, row block) work items before splitting
  pkv::MfmaShape shp;
  if (kernel != pkv::KERNEL_GENERIC && kernel_shape(kernel, &shp)) {
    tile_tokens = shp.tile_tokens;
    rows_per_block = shp.rows_per_block;
    threads = shp.threads;
    const int64_t rb = std::max<int64_t>(1, (rows_per_kv + rows_per_block - 1) / rows_per_block);
    units = (int64_t)a->batch * a->num_kv_heads * rb;
    info->grid_y = (int32_t)(a->num_kv_heads * rb);
    info->grid_z = a->batch;
  } else {
    units = total_rows * a->num_qo_heads;
    info->grid_x = (int32_t)total_rows;
    info->grid_y = a->num_qo_heads;
  }

  // Balanced decode schedule (GQA families, rows of a KV head in one block):
  // used when the units cannot fill the CUs, or on request (num_splits == -1).
  const bool gqa = is_gqa_family(kernel);
  if (a->num_splits == -1 || (a->num_splits == 0 && gqa && units < num_cus)) {
    if (!gqa || is_context)
      return fail(PKV_ERR_UNSUPPORTED, "the balanced schedule needs a GQA decode kernel family");
    // page list (and the V list), prefix, flag
    const int64_t extra = (int64_t)a->max_pages_per_seq * (a->v_block_tables ? 2 : 1) + a->batch + 2 + 3;
    const int64_t lds = (int64_t)shp.lds_static + extra * 4;
    if (lds > 160 * 1024) {
      if (a->num_splits == -1) return fail(PKV_ERR_UNSUPPORTED, "balanced schedule: page table too wide for LDS");
    } else {
      // resident workgroups per CU: LDS-limited, and at most 8 waves per CU
      // (two per SIMD: these kernels use up to 256 VGPRs)
      const int64_t per_cu_lds = std::max<int64_t>(1, (160 * 1024) / lds);
      const int64_t per_cu_waves = std::max<int64_t>(1, shp.waves_per_cu / std::max(1, threads / 64));
      const int64_t W = (int64_t)num_cus * std::min(per_cu_lds, per_cu_waves);
      const int64_t U = (int64_t)a->batch * a->num_kv_heads;
      const int64_t slot_rows = (int64_t)a->q_len * G;
      info->schedule = 1;
      info->counter_words = (int32_t)U;
      // the fused reducer lives in the direct-to-LDS stream kernel and keeps its
      // per-unit owner table in the ring's LDS.  Every owner of a unit owns at least
      // one of its pages, and the kernels clamp a request to the table width, so
      // a unit has at most min(W, max_pages_per_seq) owners.
      const int64_t owners = std::min<int64_t>(W, std::max<int64_t>(a->max_pages_per_seq, 1));
      const bool fits = owners <= (int64_t)shp.lds_static / 4;
      info->fused_merge = a->merge_counters != nullptr && is_ring(kernel) && fits;
      info->num_splits = (int32_t)(W + U);
      info->pages_per_split = 0;
      info->grid_x = (int32_t)W;
      info->grid_y = info->grid_z = 1;
      info->block_threads = threads;
      info->workspace_bytes = (size_t)(W + U) * slot_rows * (size_t)(a->head_dim_v + 1) * sizeof(float) +
                              (size_t)(a->batch + 1) * sizeof(int32_t) + 3 * 256;
      return PKV_OK;
    }
  }

  // Split-KV sizing.  When the (request, KV head, row block) units already
  // fill the CUs, one partition per unit streams each request's pages once and
  // needs no reducer.  Otherwise cut every unit into page-aligned partitions so
  // the longest request yields about four partitions per CU: the planner only
  // knows max_kv_len, so shorter requests simply own fewer live partitions
  // (the rest exit at once and are never merged).  When a unit has more than
  // 16 packed rows (context, MLA), each partition writes and the reducer reads
  // back fp32 partial rows for all of them, so such plans take only the
  // partitions that fill the CUs once.  Measured on MI355X: one request of 511
  // rows over 2047 keys (Hq 64 / Hkv 8): 80.7 us unsplit, 71.1 us with 2
  // partitions, 85.4 with 4, 122.6 with 8; MLA decode of 64 requests over
  // 4096 keys: 537 / 298 / 206 / 240 / 300 us with 1 / 2 / 4 / 8 / 16; of 16
  // requests over 16384 keys: 200 us with 16 partitions, 294 with 64.
  int S = std::max(a->num_splits, 0);
  int64_t pps;
  if (S == 0) {
    if (units >= num_cus) {
      S = 1;
    } else {
      const int64_t per_cu = (is_context || rows_per_kv > 16) ? 1 : 4;
      const int64_t want = (per_cu * (int64_t)num_cus + units - 1) / std::max<int64_t>(units, 1);
      const int64_t min_pages = std::max<int64_t>(1, (tile_tokens + a->page_size - 1) / a->page_size);
      const int64_t s_cap = std::max<int64_t>(1, max_pages / min_pages);
      S = (int)std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(want, s_cap), kMaxSplits));
    }
  }
  pps = std::max<int64_t>(1, (max_pages + S - 1) / S);
  // round partitions up to whole tiles when pages are smaller than a tile
  if (a->page_size < tile_tokens) {
    const int64_t ppt = tile_tokens / a->page_size;
    pps = (pps + ppt - 1) / ppt * ppt;
  }
  if (kernel != pkv::KERNEL_GENERIC) {
    // the partition's page list sits in LDS after the KV stages: keep the total within 160 KiB
    const int64_t lds_room = ((int64_t)(160 * 1024 - shp.lds_static) / 4 - 8) / (a->v_block_tables ? 2 : 1);
    int64_t cap_pages = std::min<int64_t>(kMaxPagesPerSplit, lds_room);
    if (page_list_in_registers(kernel))
      cap_pages = std::min<int64_t>(cap_pages, pkv::kM32MaxPages);
    if (cap_pages < 1) return fail(PKV_ERR_UNSUPPORTED, "no LDS left for the page list");
    if (pps > cap_pages) pps = cap_pages;
  }
  S = (int)std::max<int64_t>(1, (max_pages + pps - 1) / pps);
  if (a->num_splits > 0 && S < a->num_splits) S = a->num_splits;  // honour an explicit request
  if (S > kMaxSplits) return fail(PKV_ERR_UNSUPPORTED, "plan needs %d partitions (max %d)", S, kMaxSplits);

  info->num_splits = S;
  info->pages_per_split = (int32_t)pps;
  info->block_threads = threads;
  if (kernel == pkv::KERNEL_GENERIC) {
    info->grid_z = S;
  } else {
    info->grid_x = S;
  }
  info->workspace_bytes =
      S > 1 ? (size_t)S * (size_t)total_rows * a->num_qo_heads * (size_t)(a->head_dim_v + 1) * sizeof(float) + 256
            : 0;
  return PKV_OK;
}

pkv_status run(const pkv_args* a, bool is_context, void* ws, size_t ws_bytes, void* stream) {
  int dev = 0, cus = 256;
  pkv_plan_info plan;
  // CU count of the current device sizes the plan (host query, no device sync)
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  pkv_status st = make_plan(a, is_context, cus, &plan);
  if (st != PKV_OK) return st;
  if (a->batch == 0) return ok();
  if (plan.workspace_bytes > 0) {
    if (!ws || ws_bytes < plan.workspace_bytes)
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", plan.workspace_bytes, ws_bytes);
  }
  const int G = a->num_qo_heads / a->num_kv_heads;
  const int64_t total_rows = is_context ? a->total_q : (int64_t)a->batch * a->q_len;

  pkv::KParams p;
  std::memset(&p, 0, sizeof p);
  p.batch = a->batch;
  p.q_len = is_context ? 0 : a->q_len;
  p.num_qo_heads = a->num_qo_heads;
  p.num_kv_heads = a->num_kv_heads;
  p.group = G;
  p.head_dim_qk = a->head_dim_qk;
  p.head_dim_v = a->head_dim_v;
  p.page_size = a->page_size;
  p.log2_page = is_pow2(a->page_size) ? ilog2(a->page_size) : 0;
  p.max_pages_per_seq = a->max_pages_per_seq;
  p.num_pages = a->num_pages;
  p.is_context = is_context ? 1 : 0;
  p.causal = a->causal ? 1 : 0;
  p.num_splits = plan.num_splits;
  p.pages_per_split = plan.pages_per_split;
  p.row_blocks = 1;
  if (plan.kernel != pkv::KERNEL_GENERIC) p.row_blocks = plan.grid_y / a->num_kv_heads;
  p.total_q = is_context ? a->total_q : a->batch * a->q_len;
  p.max_q_len = is_context ? a->max_q_len : a->q_len;
  p.q_dtype = a->q_dtype;
  p.kv_dtype = a->kv_dtype;
  p.o_dtype = a->o_dtype;
  p.q = a->q;
  p.k = a->k_pages;
  p.v = a->v_shares_k ? a->k_pages : a->v_pages;
  p.table = a->block_tables;
  p.seq_lens = a->seq_lens;
  p.q_indptr = is_context ? a->q_indptr : nullptr;
  p.out = a->out;
  p.lse_out = a->lse_out;
  p.err_word = a->err_word;
  p.k_scale_dev = a->k_scale_dev;
  p.v_scale_dev = a->v_scale_dev;
  p.q_st = a->q_stride_tok;
  p.q_sh = a->q_stride_head;
  p.o_st = a->o_stride_tok;
  p.o_sh = a->o_stride_head;
  p.k_sp = a->k_stride_page;
  p.k_sh = a->k_stride_head;
  p.k_stok = a->k_stride_tok;
  p.v_sp = a->v_shares_k ? a->k_stride_page : a->v_stride_page;
  p.v_sh = a->v_shares_k ? a->k_stride_head : a->v_stride_head;
  p.v_stok = a->v_shares_k ? a->k_stride_tok : a->v_stride_tok;
  p.table_stride = a->table_stride;
  p.rows_total = total_rows * a->num_qo_heads;
  p.scale = a->scale;
  p.k_scale = a->k_scale;
  p.v_scale = a->v_scale;
  p.sinks = a->sinks;
  p.v_table = a->v_block_tables;
  p.page_list_cap = plan.pages_per_split;
  p.max_kv_len = a->max_kv_len;
  {
    // a split plan streams S partitions of pages_per_split pages; keys past
    // them are never read, so a longer request is cut there (and flagged)
    const int64_t cap = (int64_t)a->max_pages_per_seq * a->page_size;
    const int64_t span = plan.schedule == 1 ? cap : (int64_t)plan.num_splits * plan.pages_per_split * a->page_size;
    p.kv_span = (int32_t)std::min<int64_t>(cap, span);
  }
  if (plan.schedule == 1) {
    p.stream = 1;
    p.seg_cost = seg_cost_pages(a);
    p.num_wg = plan.grid_x;
    p.slot_rows = a->q_len * G;
    p.page_list_cap = a->max_pages_per_seq;
    const size_t n_o = (size_t)plan.num_splits * p.slot_rows * a->head_dim_v;
    const size_t n_l = (size_t)plan.num_splits * p.slot_rows;
    uintptr_t base = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
    p.ws_o = reinterpret_cast<float*>(base);
    uintptr_t lse_base = (reinterpret_cast<uintptr_t>(p.ws_o + n_o) + 255) & ~uintptr_t(255);
    p.ws_lse = reinterpret_cast<float*>(lse_base);
    uintptr_t pfx_base = (reinterpret_cast<uintptr_t>(p.ws_lse + n_l) + 255) & ~uintptr_t(255);
    p.ws_pfx = reinterpret_cast<int32_t*>(pfx_base);
    p.counters = plan.fused_merge ? a->merge_counters : nullptr;
  } else if (plan.num_splits > 1) {
    uintptr_t base = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
    p.ws_o = reinterpret_cast<float*>(base);
    p.ws_lse = p.ws_o + (size_t)plan.num_splits * p.rows_total * a->head_dim_v;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = plan.kernel == pkv::KERNEL_GENERIC         ? pkv::launch_generic(p, s)
                 : is_m32(plan.kernel)                       ? pkv::launch_m32(plan.kernel, p, s)
                 : is_mla32(plan.kernel)                     ? pkv::launch_mla32(plan.kernel, p, s)
                 : is_ring(plan.kernel)                      ? pkv::launch_dma(plan.kernel, p, s)
                                                             : pkv::launch_mfma(plan.kernel, p, s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  if (plan.num_splits > 1 && !plan.fused_merge) {
    pkv::MergeParams mp;
    std::memset(&mp, 0, sizeof mp);
    mp.num_splits = plan.num_splits;
    mp.num_qo_heads = a->num_qo_heads;
    mp.dv = a->head_dim_v;
    mp.o_dtype = a->o_dtype;
    mp.num_rows = p.rows_total;
    mp.o_st = a->o_stride_tok;
    mp.o_sh = a->o_stride_head;
    mp.o_part = p.ws_o;
    mp.lse_part = p.ws_lse;
    mp.out = a->out;
    mp.lse_out = a->lse_out;
    mp.seq_lens = a->seq_lens;
    mp.q_indptr = p.q_indptr;
    mp.batch = a->batch;
    mp.q_len = p.q_len;
    mp.causal = p.causal;
    mp.is_context = p.is_context;
    mp.split_tokens = plan.pages_per_split * a->page_size;
    mp.cap_tokens = p.kv_span;
    mp.max_kv_len = a->max_kv_len;
    mp.max_q_len = p.max_q_len;
    mp.total_q = p.total_q;
    mp.err_word = a->err_word;
    mp.sinks = a->sinks;
    mp.vec4 = a->head_dim_v % 4 == 0;  // the workspace partials are 256-byte aligned
    if (p.stream) {
      mp.stream = 1;
      mp.num_wg = p.num_wg;
      mp.num_kv_heads = a->num_kv_heads;
      mp.group = G;
      mp.slot_rows = p.slot_rows;
      mp.page_size = a->page_size;
      mp.pfx = p.ws_pfx;
      mp.seg_cost = p.seg_cost;
    }
    e = pkv::launch_merge(mp, s);
    if (e != hipSuccess) return fail(PKV_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

// ---------------------------------------------------------------- the allocation-free decode
// Scratch for pkv_decode_noalloc: the Split-KV partials, LSE slots and the
// balanced schedule's page prefix live in this array instead of a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends; host code never uses the array's name as an address (on the
// host it is only a stand-in), only the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device, looked up once per device
pkv_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_last_error(void) { return g_last_error.c_str(); }

pkv_status pkv_plan(const pkv_args* args, int is_context, int num_cus, pkv_plan_info* info) {
  if (!info) return fail(PKV_ERR_INVALID_ARG, "info is NULL");
  pkv_status st = make_plan(args, is_context != 0, num_cus, info);
  return st == PKV_OK ? ok() : st;
}

pkv_status pkv_workspace_bytes(const pkv_args* args, int is_context, size_t* bytes) {
  if (!bytes) return fail(PKV_ERR_INVALID_ARG, "bytes is NULL");
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  pkv_plan_info info;
  pkv_status st = make_plan(args, is_context != 0, cus, &info);
  if (st != PKV_OK) return st;
  *bytes = info.workspace_bytes;
  return ok();
}

pkv_status pkv_decode(const pkv_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  return run(args, false, workspace, workspace_bytes, stream);
}

pkv_status pkv_context(const pkv_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  return run(args, true, workspace, workspace_bytes, stream);
}

pkv_status pkv_decode_noalloc(const pkv_args* args, void* stream) {
  // plan first (host only): a call whose partials do not fit is refused
  // before anything touches the device
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  pkv_plan_info plan;
  pkv_status st = make_plan(args, false, cus, &plan);
  if (st != PKV_OK) return st;
  if (plan.workspace_bytes > (size_t)PKV_NOALLOC_SCRATCH_BYTES)
    return fail(PKV_ERR_WORKSPACE,
                "pkv_decode_noalloc: this call needs %zu bytes of scratch; the library's static scratch holds %zu "
                "(use pkv_decode with a caller workspace)",
                plan.workspace_bytes, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
  if (args->batch == 0) return ok();
  void* ws = nullptr;
  if (plan.workspace_bytes > 0) {
    st = scratch_for_current_device(&ws);
    if (st != PKV_OK) return st;
  }
  return run(args, false, ws, plan.workspace_bytes > 0 ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}

pkv_status pkv_lse_merge(int32_t num_splits, int32_t num_rows, int32_t num_qo_heads, int32_t head_dim_v,
                         const float* o_part, const float* lse_part, void* out, int32_t o_dtype,
                         int64_t o_stride_tok, int64_t o_stride_head, float* lse_out, void* stream) {
  if (num_splits < 1 || num_splits > kMaxSplits)
    return fail(PKV_ERR_INVALID_ARG, "num_splits must be in [1, %d]", kMaxSplits);
  if (num_rows < 0 || num_qo_heads < 1 || head_dim_v < 1 || head_dim_v > 512)
    return fail(PKV_ERR_INVALID_ARG, "need num_rows >= 0, num_qo_heads >= 1, 1 <= head_dim_v <= 512");
  if (o_dtype != PKV_DTYPE_F32 && o_dtype != PKV_DTYPE_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "o_dtype %d not supported", o_dtype);
  if (o_stride_head < head_dim_v || o_stride_tok < head_dim_v)
    return fail(PKV_ERR_INVALID_ARG, "out strides too small for head_dim_v");
  if (num_rows == 0) return ok();
  if (!o_part || !lse_part || !out) return fail(PKV_ERR_INVALID_ARG, "o_part, lse_part and out are required");
  pkv::MergeParams mp;
  std::memset(&mp, 0, sizeof mp);
  mp.num_splits = num_splits;
  mp.num_qo_heads = num_qo_heads;
  mp.dv = head_dim_v;
  mp.o_dtype = o_dtype;
  mp.num_rows = num_rows;
  mp.o_st = o_stride_tok;
  mp.o_sh = o_stride_head;
  mp.o_part = o_part;
  mp.lse_part = lse_part;
  mp.out = out;
  mp.lse_out = lse_out;
  mp.vec4 = head_dim_v % 4 == 0 && (reinterpret_cast<uintptr_t>(o_part) & 15u) == 0;
  hipError_t e = pkv::launch_merge(mp, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- paged KV append

extern "C" pkv_status pkv_append(const pkv_append_args* a, void* stream) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  if (a->num_tokens < 0 || a->batch < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens and batch must be >= 0");
  if (a->num_qo_heads < 1 || a->num_kv_heads < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_qo_heads and num_kv_heads must be >= 1");
  if (a->head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: the append route is built for 128", a->head_dim);
  if (a->page_size < 1) return fail(PKV_ERR_INVALID_ARG, "page_size must be >= 1 (got %d)", a->page_size);
  if (a->norm_policy < 0 || a->norm_policy > 2) return fail(PKV_ERR_INVALID_ARG, "norm_policy must be 0, 1 or 2");
  if (a->kv_dtype != PKV_DTYPE_BF16 && a->kv_dtype != PKV_DTYPE_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype %d: caches are bf16 or e4m3", a->kv_dtype);
  if (a->kv_dtype == PKV_DTYPE_FP8_E4M3 &&
      (!(std::fabs(a->k_scale) > 0.f) || !(std::fabs(a->v_scale) > 0.f) || !std::isfinite(a->k_scale) ||
       !std::isfinite(a->v_scale)))
    return fail(PKV_ERR_INVALID_ARG, "e4m3 caches need finite non-zero k_scale and v_scale");
  if (!(a->eps >= 0.f)) return fail(PKV_ERR_INVALID_ARG, "eps must be >= 0");
  if (a->q_quant < 0 || a->q_quant > 2) return fail(PKV_ERR_INVALID_ARG, "q_quant must be 0, 1 or 2");
  if (a->q_quant == 1) {
    if (!(a->upper_max > 0.f && a->upper_max <= 448.f))
      return fail(PKV_ERR_INVALID_ARG, "upper_max must be finite and in (0, 448]");
    if (a->q_scale_layout != 0 && a->q_scale_layout != 1)
      return fail(PKV_ERR_INVALID_ARG, "q_scale_layout must be 0 ([T, Hq]) or 1 ([B, Hq, stride])");
    if (a->q_scale_layout == 1 && a->q_scale_stride < 1)
      return fail(PKV_ERR_INVALID_ARG, "q_scale_stride must be >= 1 for the [B, Hq, stride] layout");
  }
  if (a->q_quant == 2 && (!std::isfinite(a->q_scale_inv) || a->q_scale_inv == 0.f))
    return fail(PKV_ERR_INVALID_ARG, "q_scale_inv must be finite and non-zero");
  if (a->layout != PKV_LAYOUT_HND && a->layout != PKV_LAYOUT_NHD)
    return fail(PKV_ERR_INVALID_ARG, "layout %d unknown", a->layout);
  pkv_status st = check_pool_strides(a->layout, a->num_kv_heads, a->page_size, 128, a->k_stride_page,
                                     a->k_stride_head, a->k_stride_tok, "k cache");
  if (st != PKV_OK) return st;
  st = check_pool_strides(a->layout, a->num_kv_heads, a->page_size, 128, a->v_stride_page, a->v_stride_head,
                          a->v_stride_tok, "v cache");
  if (st != PKV_OK) return st;
  if (a->batch == 0 || (a->num_tokens == 0 && !a->clear_tail)) return ok();
  if (!a->q_indptr || !a->seq_lens || !a->block_tables || !a->k_cache || !a->v_cache)
    return fail(PKV_ERR_INVALID_ARG, "q_indptr, seq_lens, block_tables and both caches are required");
  if (a->num_pages < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_pages must give the cache size: every page index is checked before a write");
  if (a->max_pages_per_seq < 1 || a->table_stride < a->max_pages_per_seq)
    return fail(PKV_ERR_INVALID_ARG, "need max_pages_per_seq >= 1 and table_stride >= max_pages_per_seq");
  if (a->num_tokens > 0) {
    if (!a->qkv || !a->cos_sin || !a->out_q) return fail(PKV_ERR_INVALID_ARG, "qkv, cos_sin and out_q are required");
    if (a->q_quant == 1 && (!a->q_scale || (reinterpret_cast<uintptr_t>(a->q_scale) & 3u)))
      return fail(PKV_ERR_INVALID_ARG, "q_quant 1 needs a 4-byte aligned q_scale");
    if (a->norm_policy != 0 && (!a->q_weight || !a->k_weight))
      return fail(PKV_ERR_INVALID_ARG, "norm_policy %d needs q_weight and k_weight", a->norm_policy);
    if (a->max_pos < 1) return fail(PKV_ERR_INVALID_ARG, "max_pos must be >= 1");
    const int64_t row = (int64_t)(a->num_qo_heads + 2 * a->num_kv_heads) * 128;
    if (a->qkv_stride_tok < row) return fail(PKV_ERR_INVALID_ARG, "qkv_stride_tok smaller than (Hq + 2 Hkv) * 128");
    const uintptr_t al = reinterpret_cast<uintptr_t>(a->qkv) |
                         (a->q_quant == 0 ? reinterpret_cast<uintptr_t>(a->out_q) : 0) |
                         reinterpret_cast<uintptr_t>(a->q_weight) | reinterpret_cast<uintptr_t>(a->k_weight);
    if ((al & 1u) || (reinterpret_cast<uintptr_t>(a->cos_sin) & 3u))
      return fail(PKV_ERR_INVALID_ARG, "bf16 arrays must be 2-byte and cos_sin 4-byte aligned");
  }
  if (a->kv_dtype == PKV_DTYPE_BF16 &&
      ((reinterpret_cast<uintptr_t>(a->k_cache) | reinterpret_cast<uintptr_t>(a->v_cache)) & 1u))
    return fail(PKV_ERR_INVALID_ARG, "bf16 caches must be 2-byte aligned");
  hipError_t e = pkv::launch_append(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "append launch failed: %s", hipGetErrorString(e));
  return ok();
}

// pkv_internal.h -- what the C-ABI layer hands to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

// Kernel families picked by the planner (reported through pkv_plan_info.kernel).
// Ids are stable: the numbers missing below belonged to tile-shape variants
// that lost to the kept families on every workload and were removed.
enum KernelId : int32_t {
  KERNEL_NONE = 0,
  KERNEL_GENERIC = 1,     // VALU, one wavefront per (query row, head, split); any dtype / head dim
  KERNEL_GQA_BF16 = 2,    // MFMA, <= 16 packed rows per KV head, D = 128, bf16 KV, register-staged tiles
  KERNEL_GQA_FP8 = 3,     // same with e4m3 KV
  KERNEL_WIDE_BF16 = 4,   // MFMA, 128 packed rows per workgroup (context / large groups), D = 128
  KERNEL_WIDE_FP8 = 5,
  KERNEL_MLA_BF16 = 6,    // MFMA, 128 heads on one latent KV head, D_qk = 576, D_v = 512
  KERNEL_MLA_FP8 = 7,
  // direct-to-LDS ring families (pkv_attn_dma.hip); KV stays in its stored dtype in LDS
  KERNEL_DMA_WIDE_BF16 = 15,
  KERNEL_DMA_WIDE_FP8 = 16,
  KERNEL_DMA_MLA_BF16 = 17,
  KERNEL_DMA_MLA_FP8 = 18,
  KERNEL_DMA_GQA_FP8_N2 = 31,   // e4m3 GQA decode: 2 token waves, 64-key tiles, 2 stages (four groups per CU)
  // 32x32x16 MFMA context (pkv_attn_m32.hip): D = 128, 8 waves x 32 rows, 2 x 64 KiB stages of 128 keys
  KERNEL_M32_CTX_W8T128 = 36,
  // MLA latent decode on 32x32x16 MFMA, 32 heads per wave, one wave per SIMD (pkv_attn_mla.hip)
  KERNEL_MLA32_BF16 = 37,
  KERNEL_COUNT = 39,
};

// Everything a kernel reads, by value.  Element strides as in pkv_args.
struct KParams {
  int32_t batch, q_len, num_qo_heads, num_kv_heads, group;
  int32_t head_dim_qk, head_dim_v, page_size, log2_page;
  int32_t max_pages_per_seq, num_pages, is_context, causal;
  int32_t num_splits, pages_per_split, row_blocks, total_q, max_q_len;
  int32_t q_dtype, kv_dtype, o_dtype, pad0;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* q_indptr;
  void* out;
  float* lse_out;
  int32_t* err_word;
  const float* k_scale_dev;
  const float* v_scale_dev;
  float* ws_o;    // [num_splits, rows_total, head_dim_v] when split
  float* ws_lse;  // [num_splits, rows_total]
  int64_t q_st, q_sh, o_st, o_sh;
  int64_t k_sp, k_sh, k_stok, v_sp, v_sh, v_stok, table_stride;
  int64_t rows_total;  // total query rows * num_qo_heads
  float scale, k_scale, v_scale, pad1;
  // balanced decode schedule (stream != 0): num_wg workgroups, partial rows
  // indexed [slot][packed row] with slot_rows packed rows per slot, and the
  // per-request page prefix written to ws_pfx for the reducer
  int32_t stream, num_wg, slot_rows, page_list_cap;
  int32_t seg_cost, pad2;  // placeholder pages charged per segment start
  // keys a request may use: seq_lens[b] is clamped to kv_span, the table
  // capacity or, for a plan of S partitions of pages_per_split pages each,
  // S * pages_per_split * page_size when that is smaller; a length above the
  // host bound max_kv_len sets PKV_DEVERR_SEQ_GT_MAXLEN
  int32_t kv_span, max_kv_len;
  int32_t* ws_pfx;
  // balanced schedule with the fused reducer: one zero-at-rest counter per
  // (request, KV head); null selects the separate reducer kernel
  int32_t* counters;
  const float* sinks;      // [num_qo_heads] sink logits, or null
  const int32_t* v_table;  // separate V page table, or null (V pages then come from `table`)
};

struct LaunchShape {
  dim3 grid;
  dim3 block;
  size_t lds_bytes;
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_generic(const KParams& p, hipStream_t s);
hipError_t launch_mfma(int32_t kernel, const KParams& p, hipStream_t s);
// Split-KV reducer arguments.  seq_lens == nullptr: every partition of every
// row is live (the standalone entry point); otherwise the request geometry
// gives each row its live partition count.
struct MergeParams {
  int32_t num_splits, num_qo_heads, dv, o_dtype;
  int64_t num_rows, o_st, o_sh;
  const float* o_part;
  const float* lse_part;
  void* out;
  float* lse_out;
  const int32_t* seq_lens;
  const int32_t* q_indptr;
  int32_t batch, q_len, causal, is_context;
  int32_t split_tokens, cap_tokens, max_q_len, total_q;  // cap_tokens = KParams::kv_span
  int32_t max_kv_len, pad_m;
  // balanced decode schedule: row (t, h) of KV head g reads slots w + b*Hkv + g
  int32_t stream, num_wg, num_kv_heads, group, slot_rows, page_size, seg_cost;
  const int32_t* pfx;
  int32_t* err_word;
  // 1: head_dim_v % 4 == 0 and o_part 16-byte aligned (partial rows read 16 bytes at a time)
  int32_t vec4;
  const float* sinks;  // [num_qo_heads] sink logits folded into each merged row, or null
  // set by launch_merge: rows merged per workgroup and thread subsets per row
  int32_t rows_per_wg, subsets;
};
hipError_t launch_merge(MergeParams mp, hipStream_t s);

// The paged KV append producer (pkv_append.hip); arguments validated by the caller.
hipError_t launch_append(const pkv_append_args* a, hipStream_t s);

// Static shape facts of the MFMA kernel families (host-side planner input).
struct MfmaShape {
  int rows_per_block;    // packed query rows per workgroup
  int tile_tokens;       // KV tokens per pipeline stage
  int threads;           // workgroup size
  size_t lds_static;     // LDS for the KV stages and reductions (page list excluded)
  int waves_per_cu = 8;  // register-limited resident waves per CU (the balanced schedule sizes its grid by it)
};
bool mfma_shape(int32_t kernel, MfmaShape* out);
bool dma_shape(int32_t kernel, MfmaShape* out);
hipError_t launch_dma(int32_t kernel, const KParams& p, hipStream_t s);
bool m32_shape(int32_t kernel, MfmaShape* out);
// the 32x32 family keeps a partition's page list in registers: at most this many pages
constexpr int kM32MaxPages = 128;
hipError_t launch_m32(int32_t kernel, const KParams& p, hipStream_t s);
bool mla32_shape(int32_t kernel, MfmaShape* out);
hipError_t launch_mla32(int32_t kernel, const KParams& p, hipStream_t s);

}  // namespace pkv

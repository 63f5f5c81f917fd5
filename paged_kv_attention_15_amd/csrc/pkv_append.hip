// pkv_append.hip -- the producer of the paged KV cache: fused QK RMSNorm +
// NeoX rotary embedding + paged K/V append, one launch (PR #5952 page,
// summary; the PR #5956 body quoted there, section "Contract").
//
// One wavefront per (packed row, head): lane l holds channels l and l + 64,
// which are exactly the pair the NeoX rotation mixes, so the rotation needs
// no data movement and the RMSNorm's sum of squares is one wavefront sum.
// Loads and stores of a head are two coalesced 128-byte (bf16) runs.  Query
// heads may leave as e4m3 codes instead (PR #5956 body, "Contract"): with a
// dynamic scale the head's absolute maximum is one more wavefront reduction.
// After the T * (Hq + 2 Hkv) row waves come B * Hkv * 2 waves that zero the
// tail of each request's last page in the K and the V cache.  Every request is
// validated on the device (lengths, q_indptr, table width, rotary table
// length, scale layout, page range) before anything of it is written.

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

struct AppendParams {
  int32_t T, B, Hq, Hkv, P, max_pages, max_pos, num_pages, policy, clear_tail, fp8;
  float eps, inv_k_scale, inv_v_scale;
  int32_t q_quant, qs_layout;
  float upper_max, q_scale_inv;
  int64_t qs_stride;
  float* q_scale;
  const uint16_t* qkv;
  int64_t qkv_st;
  const float* cos_sin;
  const uint16_t* q_w;
  const uint16_t* k_w;
  const int32_t* q_indptr;
  const int32_t* seq_lens;
  const int32_t* table;
  int64_t table_stride;
  int64_t k_sp, k_sh, k_st, v_sp, v_sh, v_st;  // cache strides (elements)
  uint16_t* out_q;
  unsigned char* k_cache;
  unsigned char* v_cache;
  int32_t* err_word;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// e4m3 code of x, round to nearest even, saturated to +-448 (finite inputs)
__device__ __forceinline__ uint8_t f32_to_e4m3_sat(float x) {
  const float c = fminf(fmaxf(x, -448.f), 448.f);
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false);
  return (uint8_t)(w & 0xFF);
}

// Validated geometry of a request given its q_indptr pair and length, or
// false (nothing of it is written).
__device__ __forceinline__ bool request_fits(const AppendParams& p, int a0, int a1, int len, int* lo, int* hi,
                                             int* L) {
  if (a0 < 0 || a1 < a0 || a1 > p.T) {
    flag_error(p.err_word, PKV_DEVERR_QINDPTR);
    return false;
  }
  if (len < a1 - a0) {
    flag_error(p.err_word, PKV_DEVERR_SEQ_LT_QLEN);
    return false;
  }
  if ((int64_t)len > (int64_t)p.max_pages * p.P) {
    flag_error(p.err_word, PKV_DEVERR_SEQ_GT_TABLE);
    return false;
  }
  if (len > p.max_pos) {
    flag_error(p.err_word, PKV_DEVERR_POS_RANGE);
    return false;
  }
  if (p.q_quant == 1 && p.qs_layout == 1 && a1 - a0 > p.qs_stride) {
    flag_error(p.err_word, PKV_DEVERR_QSCALE_ROWS);
    return false;
  }
  *lo = a0;
  *hi = a1;
  *L = len;
  return true;
}

__device__ __forceinline__ bool append_request(const AppendParams& p, int b, int* lo, int* hi, int* L) {
  return request_fits(p, p.q_indptr[b], p.q_indptr[b + 1], p.seq_lens[b], lo, hi, L);
}

__device__ __forceinline__ bool page_ok(const AppendParams& p, int pg) {
  if (p.num_pages > 0 && (pg < 0 || pg >= p.num_pages)) {
    flag_error(p.err_word, PKV_DEVERR_PAGE_RANGE);
    return false;
  }
  return true;
}

__global__ __launch_bounds__(256) void append_kernel(const AppendParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = p.Hq + 2 * p.Hkv;
  const int64_t n_rows = (int64_t)p.T * H;
  if (wid < n_rows) {
    const int r = (int)(wid / H);
    const int hh = (int)(wid % H);
    // the row's own channels first: they do not depend on which request owns it
    const uint16_t* src = p.qkv + (int64_t)r * p.qkv_st + hh * 128;
    float x0 = bf16_to_f32(src[lane]), x1 = bf16_to_f32(src[lane + 64]);
    int lo_b;  // the last request whose rows start at or before r
    int lo, hi, L;
    if (p.B < 64) {
      // one pass over the whole (q_indptr, seq_lens) table: lane k holds entry k,
      // the owner is the number of requests b >= 1 starting at or before r (the
      // table is monotone in every well-formed call; request_fits catches the
      // rest), and its entries come from lanes b and b + 1 -- one memory round
      // trip instead of a chain of dependent loads
      const int qi = lane <= p.B ? p.q_indptr[lane] : 0;
      const int sl = lane < p.B ? p.seq_lens[lane] : 0;
      lo_b = __popcll(__builtin_amdgcn_ballot_w64(lane >= 1 && lane < p.B && qi <= r));
      const int a0 = __shfl(qi, lo_b, 64), a1 = __shfl(qi, lo_b + 1, 64), len = __shfl(sl, lo_b, 64);
      if (!request_fits(p, a0, a1, len, &lo, &hi, &L)) return;
    } else {
      int lo_s = 0, hi_s = p.B - 1;
      while (lo_s < hi_s) {
        const int mid = (lo_s + hi_s + 1) >> 1;
        if (p.q_indptr[mid] <= r) lo_s = mid; else hi_s = mid - 1;
      }
      lo_b = lo_s;
      if (!append_request(p, lo_b, &lo, &hi, &L)) return;
    }
    if (r < lo || r >= hi) return;  // a row no well-formed request owns
    const int pos = r + L - hi;
    const bool is_q = hh < p.Hq, is_k = !is_q && hh < p.Hq + p.Hkv;
    if (is_q || is_k) {
      const uint16_t* wv = is_q ? p.q_w : p.k_w;
      const float* cs = p.cos_sin + (int64_t)pos * 128;
      const float c = cs[lane], s = cs[lane + 64];
      auto norm = [&]() {
        const float w0 = bf16_to_f32(wv[lane]), w1 = bf16_to_f32(wv[lane + 64]);
        const float ms = wave_sum(x0 * x0 + x1 * x1) * (1.f / 128.f);
        const float rinv = 1.f / sqrtf(ms + p.eps);
        x0 = x0 * rinv * w0;
        x1 = x1 * rinv * w1;
      };
      if (p.policy == 2) norm();
      const float y0 = x0 * c - x1 * s, y1 = x1 * c + x0 * s;
      x0 = y0;
      x1 = y1;
      if (p.policy == 1) norm();
    }
    if (is_q) {
      const int64_t qrow = ((int64_t)r * p.Hq + hh) * 128;
      if (p.q_quant == 0) {
        uint16_t* dst = p.out_q + qrow;
        dst[lane] = f32_to_bf16_rne(x0);
        dst[lane + 64] = f32_to_bf16_rne(x1);
        return;
      }
      unsigned char* dst = (unsigned char*)p.out_q + qrow;
      if (p.q_quant == 1) {
        const float amax = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
        const float sc = fmaxf(amax, 1e-6f) / p.upper_max;
        if (lane == 0) {
          const int64_t at = p.qs_layout == 0 ? (int64_t)r * p.Hq + hh
                                              : ((int64_t)lo_b * p.Hq + hh) * p.qs_stride + (r - lo);
          p.q_scale[at] = sc;
        }
        dst[lane] = f32_to_e4m3_sat(x0 / sc);
        dst[lane + 64] = f32_to_e4m3_sat(x1 / sc);
      } else {
        dst[lane] = f32_to_e4m3_sat(x0 * p.q_scale_inv);
        dst[lane + 64] = f32_to_e4m3_sat(x1 * p.q_scale_inv);
      }
      return;
    }
    const int g = is_k ? hh - p.Hq : hh - p.Hq - p.Hkv;
    const int pg = p.table[(int64_t)lo_b * p.table_stride + pos / p.P];
    if (!page_ok(p, pg)) return;
    const int64_t row = is_k ? pg * p.k_sp + g * p.k_sh + (pos % p.P) * p.k_st
                             : pg * p.v_sp + g * p.v_sh + (pos % p.P) * p.v_st;
    unsigned char* cache = is_k ? p.k_cache : p.v_cache;
    if (p.fp8) {
      const float inv = is_k ? p.inv_k_scale : p.inv_v_scale;
      cache[row + lane] = f32_to_e4m3_sat(x0 * inv);
      cache[row + lane + 64] = f32_to_e4m3_sat(x1 * inv);
    } else {
      uint16_t* dst = (uint16_t*)cache + row;
      dst[lane] = f32_to_bf16_rne(x0);
      dst[lane + 64] = f32_to_bf16_rne(x1);
    }
    return;
  }
  // ---- tail waves: (request, KV head, K or V)
  const int64_t t = wid - n_rows;
  if (!p.clear_tail || t >= (int64_t)p.B * p.Hkv * 2) return;
  const int b = (int)(t / (2 * p.Hkv));
  const int g = (int)((t / 2) % p.Hkv);
  const bool k_side = (t % 2) == 0;
  int lo, hi, L;
  if (!append_request(p, b, &lo, &hi, &L) || L <= 0) return;
  const int pg = p.table[(int64_t)b * p.table_stride + (L - 1) / p.P];
  if (!page_ok(p, pg)) return;
  unsigned char* cache = k_side ? p.k_cache : p.v_cache;
  const int64_t base = k_side ? pg * p.k_sp + g * p.k_sh : pg * p.v_sp + g * p.v_sh;
  const int64_t st = k_side ? p.k_st : p.v_st;
  for (int slot = (L - 1) % p.P + 1; slot < p.P; ++slot) {
    const int64_t row = base + slot * st;
    if (p.fp8) {
      cache[row + lane] = 0;
      cache[row + lane + 64] = 0;
    } else {
      uint16_t* dst = (uint16_t*)cache + row;
      dst[lane] = 0;
      dst[lane + 64] = 0;
    }
  }
}

hipError_t launch_append(const pkv_append_args* a, hipStream_t s) {
  AppendParams p;
  p.T = a->num_tokens;
  p.B = a->batch;
  p.Hq = a->num_qo_heads;
  p.Hkv = a->num_kv_heads;
  p.P = a->page_size;
  p.max_pages = a->max_pages_per_seq;
  p.max_pos = a->max_pos;
  p.num_pages = a->num_pages;
  p.policy = a->norm_policy;
  p.clear_tail = a->clear_tail;
  p.fp8 = a->kv_dtype == PKV_DTYPE_FP8_E4M3;
  p.eps = a->eps;
  p.inv_k_scale = p.fp8 ? 1.f / a->k_scale : 1.f;
  p.inv_v_scale = p.fp8 ? 1.f / a->v_scale : 1.f;
  p.qkv = (const uint16_t*)a->qkv;
  p.qkv_st = a->qkv_stride_tok;
  p.cos_sin = a->cos_sin;
  p.q_w = (const uint16_t*)a->q_weight;
  p.k_w = (const uint16_t*)a->k_weight;
  p.q_indptr = a->q_indptr;
  p.seq_lens = a->seq_lens;
  p.table = a->block_tables;
  p.table_stride = a->table_stride;
  p.k_sp = a->k_stride_page;
  p.k_sh = a->k_stride_head;
  p.k_st = a->k_stride_tok;
  p.v_sp = a->v_stride_page;
  p.v_sh = a->v_stride_head;
  p.v_st = a->v_stride_tok;
  p.out_q = (uint16_t*)a->out_q;
  p.k_cache = (unsigned char*)a->k_cache;
  p.v_cache = (unsigned char*)a->v_cache;
  p.err_word = a->err_word;
  p.q_quant = a->q_quant;
  p.qs_layout = a->q_scale_layout;
  p.upper_max = a->upper_max;
  p.q_scale_inv = a->q_scale_inv;
  p.qs_stride = a->q_scale_stride;
  p.q_scale = a->q_scale;
  const int64_t waves = (int64_t)p.T * (p.Hq + 2 * p.Hkv) + (p.clear_tail ? (int64_t)p.B * p.Hkv * 2 : 0);
  if (waves == 0 || p.B == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace pkv

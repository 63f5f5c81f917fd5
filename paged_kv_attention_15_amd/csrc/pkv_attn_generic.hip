// pkv_attn_generic.hip -- the complete-domain VALU kernel and the log-sum-exp reducer.
//
// attn_generic_kernel covers every argument combination the MFMA families do
// not (fp32 queries or caches, head dims other than 128 / 576+512, page sizes
// that are not powers of two, ...), the way the flashinfer.cake_fmha API page
// keeps a complete-domain component behind its optimized routes.  One wavefront
// owns one (query row, query head, Split-KV partition); per 64-key chunk:
//   lane-per-key scores (q in LDS, the key row decoded from its storage dtype),
//   a wavefront max / sum (online softmax in the exp2 domain), then
//   lane-per-channel accumulation of p_j * v_j with p broadcast through LDS.
//
// lse_merge_kernel is the Split-KV reducer (PR #4557 page: partitions merged
// by a separate reducer): per row, L* = max_s lse_s, w_s = exp(lse_s - L*)
// (empty partitions, lse = -inf, are selected out and their rows never read),
// out = sum_s w_s O_s / sum_s w_s, lse = L* + ln(sum_s w_s).

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

__device__ __forceinline__ float load_elem(const void* base, int64_t idx, int dtype) {
  if (dtype == PKV_DTYPE_F32) return ((const float*)base)[idx];
  if (dtype == PKV_DTYPE_BF16) return bf16_bits_to_f32(((const uint16_t*)base)[idx]);
  return e4m3_to_f32(((const uint8_t*)base)[idx]);
}

constexpr int kGenericMaxDqk = 1024;
constexpr int kGenericMaxDv = 512;

__global__ __launch_bounds__(64) void attn_generic_kernel(const KParams p) {
  __shared__ float s_q[kGenericMaxDqk];
  __shared__ float s_p[64];
  __shared__ int64_t s_voff[64];

  const int lane = threadIdx.x;
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int split = blockIdx.z;
  const int G = p.group;
  const int g = h / G;

  // ---- which request owns query row t
  int b, t0, n_b;
  if (p.is_context) {
    int lo = 0, hi = p.batch - 1;
    while (lo < hi) {  // last b with q_indptr[b] <= t
      int mid = (lo + hi + 1) >> 1;
      if (p.q_indptr[mid] <= t) lo = mid; else hi = mid - 1;
    }
    b = lo;
    t0 = p.q_indptr[b];
    const int a1 = p.q_indptr[b + 1];
    const bool bad = (t0 < 0) || (a1 < t0) || (a1 - t0 > p.max_q_len) || (a1 > p.total_q);
    if (bad || t < t0 || t >= a1) {
      if (bad && split == 0 && h == 0 && lane == 0) flag_error(p.err_word, PKV_DEVERR_QINDPTR);
      return;  // row owned by no well-formed request
    }
    n_b = a1 - t0;
  } else {
    b = t / p.q_len;
    t0 = b * p.q_len;
    n_b = p.q_len;
  }
  const int i = t - t0;
  int L = p.seq_lens[b];
  const int cap = p.max_pages_per_seq * p.page_size;
  if (split == 0 && h == 0 && i == 0 && lane == 0) {
    if (L > cap) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_TABLE);
    if (L > p.max_kv_len) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_MAXLEN);
    if (L < n_b) flag_error(p.err_word, PKV_DEVERR_SEQ_LT_QLEN);
  }
  L = max(0, min(L, p.kv_span));
  const int c = p.causal ? min(L, max(0, L - n_b + i + 1)) : L;
  const int kv_lo = split * p.pages_per_split * p.page_size;
  const int kv_hi = min(kv_lo + p.pages_per_split * p.page_size, c);

  if (kv_hi <= kv_lo && p.ws_o != nullptr) return;  // partition the reducer never reads

  const float k_scale = p.k_scale_dev ? *p.k_scale_dev : p.k_scale;
  const float v_scale = p.v_scale_dev ? *p.v_scale_dev : p.v_scale;
  const float sc2 = p.scale * k_scale * kLog2e;

  for (int d = lane; d < p.head_dim_qk; d += 64)
    s_q[d] = load_elem(p.q, t * p.q_st + h * p.q_sh + d, p.q_dtype);
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  float o[kGenericMaxDv / 64];
#pragma unroll
  for (int k = 0; k < kGenericMaxDv / 64; ++k) o[k] = 0.f;

  for (int j0 = kv_lo; j0 < kv_hi; j0 += 64) {
    const int tok = j0 + lane;
    const bool valid = tok < kv_hi;
    float s = -INFINITY;
    int64_t voff = 0;
    if (valid) {
      int pg = p.table[(int64_t)b * p.table_stride + tok / p.page_size];
      if (p.num_pages > 0 && (pg < 0 || pg >= p.num_pages)) {
        flag_error(p.err_word, PKV_DEVERR_PAGE_RANGE);
        pg = min(max(pg, 0), p.num_pages - 1);
      }
      const int off = tok % p.page_size;
      const int64_t koff = (int64_t)pg * p.k_sp + (int64_t)g * p.k_sh + (int64_t)off * p.k_stok;
      int vpg = pg;
      if (p.v_table) {
        vpg = p.v_table[(int64_t)b * p.table_stride + tok / p.page_size];
        if (p.num_pages > 0 && (vpg < 0 || vpg >= p.num_pages)) {
          flag_error(p.err_word, PKV_DEVERR_PAGE_RANGE);
          vpg = min(max(vpg, 0), p.num_pages - 1);
        }
      }
      voff = (int64_t)vpg * p.v_sp + (int64_t)g * p.v_sh + (int64_t)off * p.v_stok;
      float dot = 0.f;
      for (int d = 0; d < p.head_dim_qk; ++d) dot += s_q[d] * load_elem(p.k, koff + d, p.kv_dtype);
      s = dot * sc2;
    }
    const float mx = wave_max(s);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    const float pj = valid ? exp2f(s - m_use) : 0.f;
    l_run = l_run * alpha + wave_sum(pj);
    m_run = m_new;
#pragma unroll
    for (int k = 0; k < kGenericMaxDv / 64; ++k) o[k] *= alpha;
    s_p[lane] = pj;
    s_voff[lane] = voff;
    __syncthreads();
    const int n = min(64, kv_hi - j0);
    for (int jj = 0; jj < n; ++jj) {
      const float w = s_p[jj];
      const int64_t vo = s_voff[jj];
#pragma unroll
      for (int k = 0; k < kGenericMaxDv / 64; ++k) {
        const int d = lane + 64 * k;
        if (d < p.head_dim_v) o[k] += w * load_elem(p.v, vo + d, p.kv_dtype);
      }
    }
    __syncthreads();
  }

  const bool empty = !(l_run > 0.f);
  float inv = empty ? 0.f : v_scale / l_run;
  float lse = empty ? -INFINITY : (m_run * kLn2 + __logf(l_run));
  if (p.sinks && p.ws_o == nullptr) inv *= fold_sink(lse, p.sinks[h]);  // split partials: the reducer adds it
  const int64_t row_g = (int64_t)t * p.num_qo_heads + h;
  if (p.ws_o != nullptr) {
    if (lane == 0) p.ws_lse[(int64_t)split * p.rows_total + row_g] = lse;
    if (!empty) {
      float* dst = p.ws_o + ((int64_t)split * p.rows_total + row_g) * p.head_dim_v;
#pragma unroll
      for (int k = 0; k < kGenericMaxDv / 64; ++k) {
        const int d = lane + 64 * k;
        if (d < p.head_dim_v) dst[d] = o[k] * inv;
      }
    }
  } else {
    if (p.lse_out && lane == 0) p.lse_out[row_g] = lse;
#pragma unroll
    for (int k = 0; k < kGenericMaxDv / 64; ++k) {
      const int d = lane + 64 * k;
      if (d >= p.head_dim_v) continue;
      const float v = o[k] * inv;
      const int64_t oi = t * p.o_st + h * p.o_sh + d;
      if (p.o_dtype == PKV_DTYPE_BF16) {
        ((__bf16*)p.out)[oi] = (__bf16)v;
      } else {
        ((float*)p.out)[oi] = v;
      }
    }
  }
}

hipError_t launch_generic(const KParams& p, hipStream_t s) {
  int rows = p.is_context ? p.total_q : p.batch * p.q_len;
  if (rows == 0) return hipSuccess;
  dim3 grid(rows, p.num_qo_heads, p.num_splits);
  hipLaunchKernelGGL(attn_generic_kernel, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- LSE merge
// A workgroup of kMergeThreads threads merges rows_per_wg rows; each row gets
// NQ * subsets threads.  The row's value channels are cut into NQ items of CW
// channels, and the threads of one item split the partitions between them
// (partition s goes to subset s mod subsets).  Each thread walks its
// partitions with the running-max update of the online softmax (m, l and the
// channel sums rescaled whenever the max grows), loading a batch of
// partitions' LSE and partial channels before using any of them, so a row
// costs about one memory round trip per kMergeBatch partitions of a subset;
// the subsets meet in LDS.  Few partitions per row (a split context or decode
// plan) need one subset, so a workgroup takes several rows: a call with tens of
// thousands of rows then launches a few thousand workgroups, not one per row.
// An empty partition (lse = -inf, channels never written) is selected out,
// never multiplied.  With request geometry attached (decode / context calls)
// a row reads only the partitions that can hold one of its visible keys: the
// attention kernel skips the rest without writing them.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 4;

struct MergeRow {
  int live;               // partitions that may hold keys of this row
  int64_t prow0, step;    // partial row of partition s: prow0 + s * step
  int64_t w_first, TPs;   // balanced schedule: first owner workgroup and total pages (TPs = 0: unused)
  int64_t num_wg;
};

// tl: this thread's index among the NQ * S_sub threads of its row; s_red: the
// row's LDS scratch (NQ * S_sub entries of CW + 2 floats).  Every thread of the
// workgroup calls this exactly once and passes exactly one barrier in it.
template <int CW>
__device__ __forceinline__ void merge_row(const MergeParams& mp, const MergeRow& mr, const int64_t t, const int h,
                                          const bool write, float* s_red, const int tl, const int S_sub) {
  const int dv = mp.dv;
  const int NQ = (dv + CW - 1) / CW;  // items
  const int TG = NQ * S_sub;           // threads of this row (NQ >= kMergeThreads: S_sub = 1, TG = kMergeThreads)
  const int sub = NQ >= kMergeThreads ? 0 : tl / NQ;
  // balanced schedule: an owner range may hold workgroups with an empty range,
  // but only when there are fewer virtual pages than workgroups (otherwise
  // every range holds at least one page)
  const bool check_empty = mr.TPs > 0 && mr.TPs < mr.num_wg;
  auto slot_lse = [&](int s) -> float {
    if (check_empty) {
      const int64_t w = mr.w_first + s;
      if (floor_div_nonneg((w + 1) * mr.TPs, mr.num_wg) == floor_div_nonneg(w * mr.TPs, mr.num_wg))
        return -INFINITY;
    }
    return mp.lse_part[mr.prow0 + s * mr.step];
  };
  const int q0 = NQ >= kMergeThreads ? tl : tl % NQ;
  const int qstep = NQ >= kMergeThreads ? kMergeThreads : NQ;
  for (int q = q0; q < NQ; q += qstep) {
    float m = -INFINITY, l = 0.f;
    float acc[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[c] = 0.f;
    for (int s0 = sub; s0 < mr.live; s0 += S_sub * kMergeBatch) {
      float ls[kMergeBatch];
      float v[kMergeBatch][CW];
#pragma unroll
      for (int kb = 0; kb < kMergeBatch; ++kb) {
        const int s = s0 + kb * S_sub;
        const int sc = s < mr.live ? s : s0;
        ls[kb] = s < mr.live ? slot_lse(sc) : -INFINITY;
        const float* src = mp.o_part + (mr.prow0 + sc * mr.step) * dv + q * CW;
        if constexpr (CW == 4) {
          const f32x4 x = *(const f32x4*)src;
#pragma unroll
          for (int c = 0; c < 4; ++c) v[kb][c] = x[c];
        } else {
          v[kb][0] = src[0];
        }
      }
#pragma unroll
      for (int kb = 0; kb < kMergeBatch; ++kb) {
        const bool live = ls[kb] != -INFINITY;
        const float mn = live ? fmaxf(m, ls[kb]) : m;
        const float a = (m == -INFINITY) ? 0.f : __expf(m - mn);
        const float w = __expf(ls[kb] - mn);
        l = live ? l * a + w : l;
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[c] = live ? acc[c] * a + w * v[kb][c] : acc[c];
        m = mn;
      }
    }
    if (S_sub > 1) {
      float* e = s_red + (sub * NQ + q) * (CW + 2);
      e[0] = m;
      e[1] = l;
#pragma unroll
      for (int c = 0; c < CW; ++c) e[2 + c] = acc[c];
      __syncthreads();
      if (sub != 0) return;
      float M = -INFINITY;
      for (int k = 0; k < S_sub; ++k) M = fmaxf(M, s_red[(k * NQ + q) * (CW + 2)]);
      l = 0.f;
#pragma unroll
      for (int c = 0; c < CW; ++c) acc[c] = 0.f;
      if (M != -INFINITY) {
        for (int k = 0; k < S_sub; ++k) {
          const float* e = s_red + (k * NQ + q) * (CW + 2);
          const float a = e[0] == -INFINITY ? 0.f : __expf(e[0] - M);
          l += a * e[1];
#pragma unroll
          for (int c = 0; c < CW; ++c) acc[c] += a * e[2 + c];
        }
      }
      m = M;
    }
    if (!write) continue;
    float inv = l > 0.f ? 1.f / l : 0.f;
    float lse_row = (m == -INFINITY) ? -INFINITY : m + __logf(l);
    if (mp.sinks) inv *= fold_sink(lse_row, mp.sinks[h]);
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int d = q * CW + c;
      if (d >= dv) break;
      const int64_t oi = t * mp.o_st + (int64_t)h * mp.o_sh + d;
      if (mp.o_dtype == PKV_DTYPE_BF16) {
        ((__bf16*)mp.out)[oi] = (__bf16)(acc[c] * inv);
      } else {
        ((float*)mp.out)[oi] = acc[c] * inv;
      }
    }
    if (mp.lse_out && q == 0) mp.lse_out[t * mp.num_qo_heads + h] = lse_row;
  }
  if (S_sub == 1) __syncthreads();  // the one barrier of threads that merge without subsets
}

__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(const MergeParams mp) {
  __shared__ float s_red[kMergeThreads * 6];
  const int NQ = (mp.dv + (mp.vec4 ? 4 : 1) - 1) / (mp.vec4 ? 4 : 1);
  const int TG = NQ >= kMergeThreads ? kMergeThreads : NQ * mp.subsets;
  const int lr = threadIdx.x / TG;  // row of this thread inside the workgroup
  const int tl = threadIdx.x - lr * TG;
  // row indices in 32 bits (the grid's x extent times rows_per_wg stays below
  // 2^31: the host checks the row count): the 64-bit integer division
  // sequences cost more than the rest of a merged row
  const uint32_t r32 = blockIdx.x * (uint32_t)mp.rows_per_wg + (uint32_t)lr;
  const bool in_range = lr < mp.rows_per_wg && r32 < (uint32_t)mp.num_rows;
  const uint32_t nh = (uint32_t)mp.num_qo_heads;
  const uint32_t t32 = in_range ? r32 / nh : 0;
  const int64_t r = r32, t = t32;
  const int h = in_range ? (int)(r32 - t32 * nh) : 0;
  float* s_row = s_red + (lr * TG) * (mp.vec4 ? 6 : 3);

  // partial rows of this output row: `live` slots, slot k at partial row
  // prow0 + k*step (Split-KV layout: [split][row]; stream layout: a row
  // of slot (w + u) for the consecutive workgroups w that own unit u's pages)
  MergeRow mr;
  mr.live = in_range ? mp.num_splits : 0;
  mr.prow0 = r;
  mr.step = mp.num_rows;
  mr.w_first = 0;
  mr.TPs = 0;
  mr.num_wg = mp.num_wg;
  bool write = in_range;
  if (in_range && mp.stream) {
    const uint32_t ql = (uint32_t)mp.q_len;
    const int b = (int)(t32 / ql);
    const int i = (int)(t32 - (uint32_t)b * ql);
    const int g = h / mp.group;
    const int R = i * mp.group + (h % mp.group);
    if (i == 0 && h == 0 && tl == 0) {
      const int L0 = mp.seq_lens[b];
      if (L0 > mp.cap_tokens) flag_error(mp.err_word, PKV_DEVERR_SEQ_GT_TABLE);
      if (L0 > mp.max_kv_len) flag_error(mp.err_word, PKV_DEVERR_SEQ_GT_MAXLEN);
      if (L0 < mp.q_len) flag_error(mp.err_word, PKV_DEVERR_SEQ_LT_QLEN);
    }
    StreamGeom sg;
    sg.pfx = mp.pfx;
    sg.Hkv = mp.num_kv_heads;
    sg.A = mp.seg_cost;
    sg.TV = sg.request_start(mp.batch);
    sg.W = mp.num_wg;
    const int64_t npg = sg.npg(b);
    mr.live = 0;
    if (npg > 0) {
      const int64_t u = (int64_t)b * mp.num_kv_heads + g;
      const int64_t rs = sg.real(b, g);
      const int64_t w_s = sg.owner(rs);
      const int64_t w_e = sg.owner(rs + npg - 1);
      mr.live = (int)(w_e - w_s + 1);
      mr.prow0 = (w_s + u) * mp.slot_rows + R;
      mr.step = mp.slot_rows;
      mr.w_first = w_s;
      mr.TPs = sg.TV;
    }
  } else if (in_range && mp.seq_lens) {
    int b, t0, n;
    bool skip = false;
    if (mp.is_context) {
      int lo = 0, hi = mp.batch - 1;
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (mp.q_indptr[mid] <= (int)t32) lo = mid; else hi = mid - 1;
      }
      b = lo;
      t0 = mp.q_indptr[b];
      const int a1 = mp.q_indptr[b + 1];
      const bool bad = (t0 < 0) || (a1 < t0) || (a1 - t0 > mp.max_q_len) || (a1 > mp.total_q);
      skip = bad || (int)t32 < t0 || (int)t32 >= a1;  // the attention kernel skipped this row too
      n = a1 - t0;
    } else {
      b = (int)(t32 / (uint32_t)mp.q_len);
      t0 = b * mp.q_len;
      n = mp.q_len;
    }
    if (skip) {
      mr.live = 0;
      write = false;
    } else {
      const int i = (int)(t32 - t0);
      const int L = max(0, min(mp.seq_lens[b], mp.cap_tokens));
      const int c = mp.causal ? min(L, max(0, L - n + i + 1)) : L;
      mr.live = min(mp.num_splits, (c + mp.split_tokens - 1) / mp.split_tokens);
    }
  }
  if (mp.vec4) merge_row<4>(mp, mr, t, h, write, s_row, tl, mp.subsets);
  else merge_row<1>(mp, mr, t, h, write, s_row, tl, mp.subsets);
}

hipError_t launch_merge(MergeParams mp, hipStream_t s) {
  if (mp.num_rows == 0) return hipSuccess;
  // Thread subsets per row: enough that each walks about one batch of
  // partitions (the balanced schedule's rows may have many owners: all
  // threads), then as many rows per workgroup as the threads allow.
  const int NQ = (mp.dv + (mp.vec4 ? 4 : 1) - 1) / (mp.vec4 ? 4 : 1);
  const int max_sub = NQ >= kMergeThreads ? 1 : kMergeThreads / NQ;
  const int want = mp.stream ? max_sub : (mp.num_splits + kMergeBatch - 1) / kMergeBatch;
  mp.subsets = std::max(1, std::min(max_sub, want));
  const int TG = NQ >= kMergeThreads ? kMergeThreads : NQ * mp.subsets;
  mp.rows_per_wg = std::max(1, kMergeThreads / TG);
  const int64_t wgs = (mp.num_rows + mp.rows_per_wg - 1) / mp.rows_per_wg;
  hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)wgs), dim3(kMergeThreads), 0, s, mp);
  return hipGetLastError();
}

}  // namespace pkv

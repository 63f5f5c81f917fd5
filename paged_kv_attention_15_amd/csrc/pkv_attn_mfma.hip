// pkv_attn_mfma.hip -- MFMA paged attention for gfx950 (decode, MLA decode, causal context).
//
// One workgroup owns a block of packed query rows that share one KV head and
// one Split-KV partition of the request's keys:
//   packed row R (0 <= R < n_b * G) of KV head g is query row i = R / G of the
//   request and query head h = g*G + R % G, so all query heads of a GQA group
//   (flashinfer.cake_fmha API page: group-size-eight FP8 route) and the
//   speculative / context rows of the request (PR #4557 page: MTP rows; the
//   API page's q511/KV2047 context profile) ride in one tile.
//
// Pipeline per KV tile of T tokens (two LDS stages, register-staged 16-byte
// loads):
//   1. gather: every thread loads 16-byte chunks of the tile's K (and V) rows
//      through the block table (key j is token j % P of page table[j / P]),
//      converts e4m3 to bf16 when the cache is FP8, and stores them into LDS
//      with an XOR swizzle on 16-byte chunks (row r, chunk c -> c ^ (r & 15));
//   2. S^T = K * Q^T on v_mfma_f32_16x16x32_bf16: A = K rows from LDS, B = the
//      wave's Q rows held in registers.  The transposed product leaves every
//      lane with a single query row (l % 16), so the online softmax state
//      (running max m, lane-partial sum l) is per lane and the row max needs
//      only two cross-lane steps;
//   3. online softmax in the exp2 domain (scale * k_scale * log2(e) folded
//      into one multiply), masked keys selected to -inf, never multiplied;
//   4. O^T += V^T * P^T on MFMA: B = P^T straight from the softmax registers
//      (bf16), A = V^T read with ds_read_b64_tr_b16 from the same LDS tile.
// Partitions write fp32 (O / l * v_scale, natural-log LSE) to the workspace
// for the separate log-sum-exp reducer (PR #4557 page: Split-KV partitions and
// a reducer kernel); an unsplit launch writes the final output directly.
//
// Keys past the request's visible range are never loaded from their own
// address: their loads are clamped to the last visible key (a finite row),
// so NaN or stale page tails cannot reach the MFMA products.

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <int DQK_, int DV_, bool FP8_, bool VSHARE_, int RT_, int NWR_, int NWT_, int TT_, int NSTAGE_ = 2>
struct TileCfg {
  static constexpr int DQK = DQK_, DV = DV_, RT = RT_, NWR = NWR_, NWT = NWT_, TT = TT_, NSTAGE = NSTAGE_;
  static constexpr bool FP8 = FP8_, VSHARE = VSHARE_;
  static constexpr int NW = NWR * NWT;
  static constexpr int NTHR = 64 * NW;
  static constexpr int T = NWT * TT;
  static constexpr int ROWS = NWR * RT * 16;
  static constexpr int KROWB = DQK * 2;  // bf16 bytes per K row in LDS
  static constexpr int VROWB = VSHARE ? KROWB : DV * 2;
  static constexpr int KTILE = T * KROWB;
  static constexpr int VTILE = VSHARE ? 0 : T * DV * 2;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int EB = FP8 ? 1 : 2;          // source bytes per element
  static constexpr int SCK = DQK * EB / 16;       // source 16-byte chunks per K row
  static constexpr int SCV = DV * EB / 16;
  static constexpr int NLK = (T * SCK) / NTHR;
  static constexpr int NLV = VSHARE ? 0 : (T * SCV) / NTHR;
  static constexpr int NKS = DQK / 32;            // MFMA k-steps for QK
  static constexpr int NDB = DV / 16;             // 16-wide output blocks
  static constexpr int NNB = TT / 16;             // 16-token score blocks per wave
  // reduction scratch when several waves split the tile's tokens
  static constexpr int RED_O = NWT > 1 ? NW * RT * NDB * 64 * 16 : 0;
  static constexpr int RED_ML = NWT > 1 ? NW * RT * 64 * 2 * 4 : 0;
  static constexpr int LDS = (NSTAGE * STAGE > RED_O + RED_ML) ? NSTAGE * STAGE : RED_O + RED_ML;
  static_assert(NSTAGE == 1 || NSTAGE == 2, "one or two LDS stages");
  static_assert((T * SCK) % NTHR == 0, "K gather must split evenly");
  static_assert(VSHARE || (T * SCV) % NTHR == 0, "V gather must split evenly");
  static_assert(TT % 32 == 0 && DQK % 32 == 0 && DV % 16 == 0, "MFMA tiling");
  static_assert(!VSHARE || DV <= DQK, "shared V rows");
};

// swizzled byte offset of 16-byte chunk c of LDS row r (row of NC chunks)
template <int NC>
__device__ __forceinline__ int swz_chunk(int c, int r) {
  if constexpr (NC % 16 == 0) {
    return c ^ (r & 15);
  } else {
    // rows of 72 chunks (576 channels): XOR inside aligned groups of 16, the last 8 inside 8
    int m = ((c | 15) < NC) ? 15 : 7;
    return c ^ (r & m);
  }
}

template <class C>
__device__ __forceinline__ uint32_t lds_k_off(int row, int chunk) {
  return (uint32_t)(row * C::KROWB + swz_chunk<C::KROWB / 16>(chunk, row) * 16);
}
template <class C>
__device__ __forceinline__ uint32_t lds_v_off(int row, int chunk) {
  return (uint32_t)(row * C::VROWB + swz_chunk<C::VROWB / 16>(chunk, row) * 16);
}

// One piece of work: packed row block `rb` of KV head g of request b, over the
// page-aligned key range [part_lo, part_hi) (cut further at the last key any of
// its rows sees).  Writes the final rows, or a partial (O, LSE) into workspace
// slot `slot` when the call runs in Split-KV mode.  `lead` marks the piece that
// reports the request's device-side argument errors.
template <class C>
__device__ __forceinline__ void attend_block(const KParams& p, unsigned char* smem, int32_t* s_pages, const int b,
                                             const int g, const int rb, const int part_lo, const int part_hi,
                                             const int slot, const bool lead) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr = wave / C::NWT;  // row wave
  const int wt = wave % C::NWT;  // token wave
  const int tid = threadIdx.x;
  const int G4 = lane >> 4;      // 16-lane group
  const int l16 = lane & 15;
  const int G = p.group;

  __syncthreads();  // LDS of a previous piece (stream schedule) is free again

  // ---- request geometry (device values are clamped, never trusted for addressing)
  int t0, n_b;
  if (p.is_context) {
    int a0 = p.q_indptr[b], a1 = p.q_indptr[b + 1];
    bool bad = (a0 < 0) || (a1 < a0) || (a1 - a0 > p.max_q_len) || (a1 > p.total_q);
    if (bad) {
      if (lead && g == 0 && rb == 0 && tid == 0) flag_error(p.err_word, PKV_DEVERR_QINDPTR);
      return;
    }
    t0 = a0;
    n_b = a1 - a0;
  } else {
    t0 = b * p.q_len;
    n_b = p.q_len;
  }
  const int row_space = n_b * G;
  const int row0 = rb * C::ROWS;
  if (row0 >= row_space) return;  // no rows of this block exist

  int L = p.seq_lens[b];
  const int cap = p.max_pages_per_seq * p.page_size;
  if (lead && g == 0 && rb == 0 && tid == 0) {
    if (L > cap) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_TABLE);
    if (L > p.max_kv_len) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_MAXLEN);
    if (L < n_b) flag_error(p.err_word, PKV_DEVERR_SEQ_LT_QLEN);
  }
  L = max(0, min(L, p.kv_span));

  // keys this workgroup may need: its partition, cut at the last key any of its rows sees
  const int last_row = min(row0 + C::ROWS, row_space) - 1;
  const int i_max = last_row / G;
  const int c_max = p.causal ? min(L, max(0, L - n_b + i_max + 1)) : L;
  const int kv_lo = part_lo;
  const int kv_hi = min(part_hi, c_max);
  const int n_tiles = kv_hi > kv_lo ? (kv_hi - kv_lo + C::T - 1) / C::T : 0;
  // a partition past every row's visible keys: the reducer never reads it
  if (n_tiles == 0 && p.ws_o != nullptr) return;

  // ---- page list of the partition -> LDS (clamped to the pool)
  const int pg_lo = kv_lo >> p.log2_page;
  const int n_pg = n_tiles > 0 ? ((kv_hi - 1) >> p.log2_page) - pg_lo + 1 : 0;
  // a separate V table (API page, context profile with separate K/V page
  // tables) gets its own list right after the K list
  int32_t* s_vpages = p.v_table ? s_pages + p.page_list_cap : s_pages;
  for (int i = tid; i < n_pg; i += C::NTHR) {
    int pg = p.table[(int64_t)b * p.table_stride + pg_lo + i];
    if (p.num_pages > 0 && (pg < 0 || pg >= p.num_pages)) {
      flag_error(p.err_word, PKV_DEVERR_PAGE_RANGE);
      pg = min(max(pg, 0), p.num_pages - 1);
    }
    s_pages[i] = pg;
    if (p.v_table) {
      int vpg = p.v_table[(int64_t)b * p.table_stride + pg_lo + i];
      if (p.num_pages > 0 && (vpg < 0 || vpg >= p.num_pages)) {
        flag_error(p.err_word, PKV_DEVERR_PAGE_RANGE);
        vpg = min(max(vpg, 0), p.num_pages - 1);
      }
      s_vpages[i] = vpg;
    }
  }

  // ---- this lane's query rows: one per row tile
  const float k_scale = p.k_scale_dev ? *p.k_scale_dev : p.k_scale;
  const float v_scale = p.v_scale_dev ? *p.v_scale_dev : p.v_scale;
  const float sc2 = p.scale * k_scale * kLog2e;

  int row_t[C::RT], row_h[C::RT], row_c[C::RT], row_R[C::RT];
  bool row_ok[C::RT];
  bf16x8 qB[C::RT][C::NKS];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    const int R = row0 + (wr * C::RT + rt) * 16 + l16;
    row_R[rt] = R;
    row_ok[rt] = R < row_space;
    const int i = row_ok[rt] ? R / G : 0;
    row_t[rt] = t0 + i;
    row_h[rt] = g * G + (row_ok[rt] ? R % G : 0);
    int c = p.causal ? L - n_b + i + 1 : L;
    row_c[rt] = row_ok[rt] ? min(max(c, 0), kv_hi) : 0;
    const __bf16* qrow = (const __bf16*)p.q + row_t[rt] * p.q_st + row_h[rt] * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      if (row_ok[rt]) {
        qB[rt][ks] = *(const bf16x8*)(qrow + ks * 32 + G4 * 8);
      } else {
        qB[rt][ks] = bf16x8{};
      }
    }
  }

  // smallest visible-key bound over this wave's real rows: slices below it need no mask
  int c_lo = INT_MAX;
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
    if (row_ok[rt]) c_lo = min(c_lo, row_c[rt]);
  c_lo = -wave_max_i(-c_lo);
  float m_run[C::RT], l_run[C::RT];
  f32x4 O[C::RT][C::NDB];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) O[rt][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  __syncthreads();  // page list visible

  // ---- gather helpers
  const unsigned char* kbase = (const unsigned char*)p.k;
  const unsigned char* vbase = (const unsigned char*)p.v;
  u32x4 kreg[C::NLK];
  u32x4 vreg[C::NLV > 0 ? C::NLV : 1];
  const int pmask = p.page_size - 1;

  auto gather = [&](int tile) {
    const int tok0 = kv_lo + tile * C::T;
#pragma unroll
    for (int i = 0; i < C::NLK; ++i) {
      const int q = tid + i * C::NTHR;
      const int r = q / C::SCK;
      const int sc = q % C::SCK;
      const int tok = min(tok0 + r, kv_hi - 1);
      const int pg = s_pages[(tok >> p.log2_page) - pg_lo];
      const int64_t off = (int64_t)pg * p.k_sp + (int64_t)g * p.k_sh + (int64_t)(tok & pmask) * p.k_stok;
      kreg[i] = __builtin_nontemporal_load((const u32x4*)(kbase + off * C::EB + sc * 16));
    }
#pragma unroll
    for (int i = 0; i < C::NLV; ++i) {
      const int q = tid + i * C::NTHR;
      const int r = q / C::SCV;
      const int sc = q % C::SCV;
      const int tok = min(tok0 + r, kv_hi - 1);
      const int pg = s_vpages[(tok >> p.log2_page) - pg_lo];
      const int64_t off = (int64_t)pg * p.v_sp + (int64_t)g * p.v_sh + (int64_t)(tok & pmask) * p.v_stok;
      vreg[i] = __builtin_nontemporal_load((const u32x4*)(vbase + off * C::EB + sc * 16));
    }
  };

  auto stash = [&](int stage) {
    unsigned char* kst = smem + stage * C::STAGE;
    unsigned char* vst = kst + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::NLK; ++i) {
      const int q = tid + i * C::NTHR;
      const int r = q / C::SCK;
      const int sc = q % C::SCK;
      if constexpr (C::FP8) {
        u32x4 lo, hi;
        e4m3x16_to_bf16x16(kreg[i], lo, hi);
        *(u32x4*)(kst + lds_k_off<C>(r, 2 * sc)) = lo;
        *(u32x4*)(kst + lds_k_off<C>(r, 2 * sc + 1)) = hi;
      } else {
        *(u32x4*)(kst + lds_k_off<C>(r, sc)) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::NLV; ++i) {
      const int q = tid + i * C::NTHR;
      const int r = q / C::SCV;
      const int sc = q % C::SCV;
      if constexpr (C::FP8) {
        u32x4 lo, hi;
        e4m3x16_to_bf16x16(vreg[i], lo, hi);
        *(u32x4*)(vst + lds_v_off<C>(r, 2 * sc)) = lo;
        *(u32x4*)(vst + lds_v_off<C>(r, 2 * sc + 1)) = hi;
      } else {
        *(u32x4*)(vst + lds_v_off<C>(r, sc)) = vreg[i];
      }
    }
  };

  if (n_tiles > 0) {
    gather(0);
    stash(0);
  }
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int stage = C::NSTAGE == 2 ? (tile & 1) : 0;
    if (tile + 1 < n_tiles) gather(tile + 1);

    const unsigned char* kst = smem + stage * C::STAGE;
    const unsigned char* vst = C::VSHARE ? kst : kst + C::KTILE;
    const int tok_w = kv_lo + tile * C::T + wt * C::TT;  // first key of this wave's slice

    // ---- S^T = K Q^T
    f32x4 acc[C::RT][C::NNB];
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
      for (int nb = 0; nb < C::NNB; ++nb) acc[rt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
      for (int nb = 0; nb < C::NNB; ++nb) {
        const int r = wt * C::TT + nb * 16 + l16;
        const bf16x8 a = *(const bf16x8*)(kst + lds_k_off<C>(r, ks * 4 + G4));
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) acc[rt][nb] = mfma16x16x32(a, qB[rt][ks], acc[rt][nb]);
      }
    }

    // ---- online softmax (exp2 domain); keys past a row's bound are selected to -inf,
    // which only slices reaching past the wave's smallest bound need
    const bool full_slice = tok_w + C::TT <= c_lo;
    float pr[C::RT][C::NNB][4];
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < C::NNB; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = acc[rt][nb][e] * sc2;
          if (full_slice) {
            pr[rt][nb][e] = s;
          } else {
            const int tok = tok_w + nb * 16 + G4 * 4 + e;
            pr[rt][nb][e] = (tok < row_c[rt]) ? s : -INFINITY;
          }
          mx = fmaxf(mx, pr[rt][nb][e]);
        }
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const float m_new = fmaxf(m_run[rt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[rt] - m_use);
      float ps = 0.f;
#pragma unroll
      for (int nb = 0; nb < C::NNB; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pr[rt][nb][e] = fast_exp2(pr[rt][nb][e] - m_use);
          ps += pr[rt][nb][e];
        }
      l_run[rt] = l_run[rt] * alpha + ps;
      m_run[rt] = m_new;
      // alpha is exactly 1 wherever the running max did not move: rescale only if some lane's did
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) O[rt][d] *= alpha;
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int j = 0; j < C::TT / 32; ++j) {
      bf16x8 pb[C::RT];
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) {
        u32x4 w{pack_bf16x2(pr[rt][2 * j][0], pr[rt][2 * j][1]), pack_bf16x2(pr[rt][2 * j][2], pr[rt][2 * j][3]),
                pack_bf16x2(pr[rt][2 * j + 1][0], pr[rt][2 * j + 1][1]),
                pack_bf16x2(pr[rt][2 * j + 1][2], pr[rt][2 * j + 1][3])};
        pb[rt] = __builtin_bit_cast(bf16x8, w);
      }
      const int vr1 = wt * C::TT + 32 * j + 4 * G4 + (l16 >> 2);
      const int vr2 = vr1 + 16;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int ch = 2 * db + ((l16 & 3) >> 1);
        const int half = (l16 & 1) * 8;
        const s16x4 lo = lds_read_tr16(vst + lds_v_off<C>(vr1, ch) + half);
        const s16x4 hi = lds_read_tr16(vst + lds_v_off<C>(vr2, ch) + half);
        typedef short s16x8 __attribute__((ext_vector_type(8)));
        const s16x8 a8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) O[rt][db] = mfma16x16x32(a, pb[rt], O[rt][db]);
      }
    }

    if constexpr (C::NSTAGE == 2) {
      if (tile + 1 < n_tiles) stash(stage ^ 1);
      __syncthreads();
    } else {
      if (tile + 1 < n_tiles) {
        __syncthreads();  // every wave is done reading the stage
        stash(0);
        __syncthreads();
      }
    }
  }

  // ---- full row sums (the 4 lanes of a row hold partial sums)
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    l_run[rt] = xor_sum(l_run[rt], 16);
    l_run[rt] = xor_sum(l_run[rt], 32);
  }

  // ---- combine token waves (they saw disjoint key slices of the same rows)
  int db_first = 0, db_step = 1;
  if constexpr (C::NWT > 1) {
    float* red_ml = (float*)smem;                         // [NW][RT][64][2]
    f32x4* red_o = (f32x4*)(smem + C::RED_ML);            // [NW][RT][NDB][64]
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      red_ml[((wave * C::RT + rt) * 64 + lane) * 2 + 0] = m_run[rt];
      red_ml[((wave * C::RT + rt) * 64 + lane) * 2 + 1] = l_run[rt];
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) red_o[((wave * C::RT + rt) * C::NDB + d) * 64 + lane] = O[rt][d];
    }
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      float mw[C::NWT], M = -INFINITY;
#pragma unroll
      for (int w = 0; w < C::NWT; ++w) {
        mw[w] = red_ml[(((wr * C::NWT + w) * C::RT + rt) * 64 + lane) * 2 + 0];
        M = fmaxf(M, mw[w]);
      }
      const float M_use = (M == -INFINITY) ? 0.f : M;
      float lsum = 0.f;
      float wgt[C::NWT];
#pragma unroll
      for (int w = 0; w < C::NWT; ++w) {
        wgt[w] = fast_exp2(mw[w] - M_use);
        lsum += wgt[w] * red_ml[(((wr * C::NWT + w) * C::RT + rt) * 64 + lane) * 2 + 1];
      }
      m_run[rt] = M;
      l_run[rt] = lsum;
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) {
        if (d % C::NWT != wt) continue;
        f32x4 acc_o{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < C::NWT; ++w)
          acc_o += wgt[w] * red_o[(((wr * C::NWT + w) * C::RT + rt) * C::NDB + d) * 64 + lane];
        O[rt][d] = acc_o;
      }
    }
    db_first = wt;
    db_step = C::NWT;
  }

  // ---- epilogue
  const bool split_mode = p.ws_o != nullptr;
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    if (!row_ok[rt]) continue;
    const bool empty = !(l_run[rt] > 0.f);
    float inv = empty ? 0.f : v_scale / l_run[rt];
    float lse = empty ? -INFINITY : (m_run[rt] * kLn2 + __logf(l_run[rt]));
    if (p.sinks && !split_mode) inv *= fold_sink(lse, p.sinks[row_h[rt]]);  // split: the reducer adds it
    const int64_t row_g = (int64_t)row_t[rt] * p.num_qo_heads + row_h[rt];
    if (split_mode) {
      const int64_t prow = p.stream ? (int64_t)slot * p.slot_rows + row_R[rt] : (int64_t)slot * p.rows_total + row_g;
      if (G4 == 0 && db_first == 0) p.ws_lse[prow] = lse;
      if (!empty) {
        float* dst = p.ws_o + prow * C::DV + G4 * 4;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
          if (C::NWT > 1 && d % C::NWT != db_first) continue;
          *(f32x4*)(dst + d * 16) = O[rt][d] * inv;
        }
      }
    } else {
      if (p.lse_out && G4 == 0 && db_first == 0) p.lse_out[row_g] = lse;
      if (p.o_dtype == PKV_DTYPE_BF16) {
        __bf16* dst = (__bf16*)p.out + row_t[rt] * p.o_st + row_h[rt] * p.o_sh + G4 * 4;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
          if (C::NWT > 1 && d % C::NWT != db_first) continue;
          const f32x4 v = O[rt][d] * inv;
          u32x2 w{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(dst + d * 16) = w;
        }
      } else {
        float* dst = (float*)p.out + row_t[rt] * p.o_st + row_h[rt] * p.o_sh + G4 * 4;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
          if (C::NWT > 1 && d % C::NWT != db_first) continue;
          *(f32x4*)(dst + d * 16) = O[rt][d] * inv;
        }
      }
    }
  }
  (void)db_step;
}

// Per-partition grid: (partition, KV head x row block, request).
template <class C>
__global__ __launch_bounds__(C::NTHR) void attn_mfma_kernel(const KParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pages = (int32_t*)(smem + C::LDS);
  const int split = blockIdx.x;
  const int span = p.pages_per_split * p.page_size;
  attend_block<C>(p, smem, s_pages, blockIdx.z, blockIdx.y / p.row_blocks, blockIdx.y % p.row_blocks,
                  split * span, split * span + span, split, split == 0);
}

// Balanced decode schedule.  The page streams of all (request, KV head) units,
// laid end to end in the virtual page space of StreamGeom (unit u = b*Hkv + g
// owns ceil(L_b/P) pages after A placeholder pages), are cut into gridDim.x
// equal ranges, one per workgroup.  Every maximal piece of one unit's pages
// inside one workgroup's range is a segment; segment (w, u) writes its
// partial rows to workspace slot w + u, which is unique because moving from
// one segment to the next increases w or u.  The reducer recovers a row's
// segments from the same arithmetic (StreamGeom::owner).
template <class C>
__global__ __launch_bounds__(C::NTHR) void attn_mfma_stream_kernel(const KParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pages = (int32_t*)(smem + C::LDS);
  // [batch + 1] page prefix over requests, after the page list(s)
  int32_t* s_pfx = s_pages + p.page_list_cap * (p.v_table ? 2 : 1);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = p.batch;
  if (tid < 64) {
    int carry = 0;
    if (lane == 0) s_pfx[0] = 0;
    for (int c0 = 0; c0 < B; c0 += 64) {
      const int bb = c0 + lane;
      int v = 0;
      if (bb < B) {
        const int L = max(0, min(p.seq_lens[bb], p.kv_span));
        v = (L + p.page_size - 1) >> p.log2_page;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
      }
      if (bb < B) s_pfx[bb + 1] = carry + v;
      carry += __shfl(v, 63, 64);
    }
  }
  __syncthreads();
  const int Hkv = p.num_kv_heads;
  StreamGeom sg;
  sg.pfx = s_pfx;
  sg.Hkv = Hkv;
  sg.A = p.seg_cost;
  sg.TV = sg.request_start(B);
  sg.W = gridDim.x;
  const int64_t W = sg.W;
  const int64_t w = blockIdx.x;
  if (w == 0)
    for (int i = tid; i <= B; i += C::NTHR) p.ws_pfx[i] = s_pfx[i];
  int64_t pos = w * sg.TV / W;
  const int64_t end = (w + 1) * sg.TV / W;
  while (pos < end) {
    int lo = 0, hi = B - 1;  // the last request whose units start at or before pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sg.request_start(mid) <= pos) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int64_t npg = sg.npg(b);
    const int g = (int)((pos - sg.request_start(b)) / (npg + sg.A));
    const int64_t rs = sg.real(b, g);
    const int64_t seg_lo = max(pos, rs), seg_hi = min(end, rs + npg);
    if (seg_lo < seg_hi) {
      const int a = (int)(seg_lo - rs), e = (int)(seg_hi - rs);
      attend_block<C>(p, smem, s_pages, b, g, 0, a * p.page_size, e * p.page_size, (int)(w + b * Hkv + g),
                      a == 0);
    }
    pos = rs + npg;
  }
}

// ---------------------------------------------------------------- instances
using CfgGqaBf16 = TileCfg<128, 128, false, false, 1, 1, 4, 32>;
using CfgGqaFp8 = TileCfg<128, 128, true, false, 1, 1, 4, 64, 1>;
using CfgWideBf16 = TileCfg<128, 128, false, false, 2, 4, 1, 64>;
using CfgWideFp8 = TileCfg<128, 128, true, false, 2, 4, 1, 64>;
using CfgMlaBf16 = TileCfg<576, 512, false, true, 2, 4, 1, 32>;
using CfgMlaFp8 = TileCfg<576, 512, true, true, 2, 4, 1, 64>;

template <class C>
static void fill_shape(MfmaShape* s) {
  s->rows_per_block = C::ROWS;
  s->tile_tokens = C::T;
  s->threads = C::NTHR;
  s->lds_static = C::LDS;
}

bool mfma_shape(int32_t kernel, MfmaShape* s) {
  switch (kernel) {
    case KERNEL_GQA_BF16: fill_shape<CfgGqaBf16>(s); return true;
    case KERNEL_GQA_FP8: fill_shape<CfgGqaFp8>(s); return true;
    case KERNEL_WIDE_BF16: fill_shape<CfgWideBf16>(s); return true;
    case KERNEL_WIDE_FP8: fill_shape<CfgWideFp8>(s); return true;
    case KERNEL_MLA_BF16: fill_shape<CfgMlaBf16>(s); return true;
    case KERNEL_MLA_FP8: fill_shape<CfgMlaFp8>(s); return true;
    default: return false;
  }
}

template <class C>
static hipError_t launch_cfg(const KParams& p, hipStream_t s) {
  static bool attr_done = false;  // idempotent; a race only repeats the same calls
  const size_t extra = (size_t)p.page_list_cap * (p.v_table ? 2 : 1) + (p.stream ? (size_t)p.batch + 1 : 0);
  const size_t lds = C::LDS + ((extra + 3) & ~size_t(3)) * sizeof(int32_t);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mfma_kernel<C>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)attn_mfma_stream_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  if (p.stream) {
    hipLaunchKernelGGL(attn_mfma_stream_kernel<C>, dim3(p.num_wg), dim3(C::NTHR), lds, s, p);
  } else {
    dim3 grid(p.num_splits, p.num_kv_heads * p.row_blocks, p.batch);
    hipLaunchKernelGGL(attn_mfma_kernel<C>, grid, dim3(C::NTHR), lds, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_mfma(int32_t kernel, const KParams& p, hipStream_t s) {
  switch (kernel) {
    case KERNEL_GQA_BF16: return launch_cfg<CfgGqaBf16>(p, s);
    case KERNEL_GQA_FP8: return launch_cfg<CfgGqaFp8>(p, s);
    case KERNEL_WIDE_BF16: return launch_cfg<CfgWideBf16>(p, s);
    case KERNEL_WIDE_FP8: return launch_cfg<CfgWideFp8>(p, s);
    case KERNEL_MLA_BF16: return launch_cfg<CfgMlaBf16>(p, s);
    case KERNEL_MLA_FP8: return launch_cfg<CfgMlaFp8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv

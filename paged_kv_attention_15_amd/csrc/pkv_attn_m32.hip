// pkv_attn_m32.hip -- paged attention on v_mfma_f32_32x32x16_bf16 for the
// compute-heavy context shape: causal context over a GQA group (the MLA
// latent decode on the same instruction lives in pkv_attn_mla.hip).
//
// Measured on gfx950, the 32x32x16 bf16 MFMA sustains one instruction per 32
// cycles per SIMD from a single wave (the full bf16 matrix rate), while
// back-to-back 16x16x32 instructions reach about half of it; so the products
// that dominate this shape use the 32x32 form.  Both are transposed, putting
// the query rows on the column axis of the MFMA:
//   S^T[keys x rows] = K[keys x d] Q^T[d x rows]          A = K rows (LDS), B = Q (registers)
//   O^T[dv x rows]  += V^T[dv x keys] P^T[keys x rows]    A = V^T (LDS transpose reads), B = P
// Operand element e of lane l is (row or column l%32, k 8(l/32)+e); result
// element e of lane l is (row 8(e/4) + 4(l/32) + e%4, column l%32).  A row r of
// the S^T product is fed the key whose index is r with bits 2 and 3 exchanged;
// result elements 8s..8s+7 of lane l then hold keys 16s + 8(l/32) + 0..7, which
// is exactly the B operand of the s-th 16-key step of the PV product: P^T goes
// from the softmax to the second product without crossing lanes.
//
// Each wave owns RB blocks of 32 packed query rows (RB > 1 re-uses every K and
// V^T operand read from LDS for RB products, which is what keeps LDS traffic
// below the MFMA time).  KV tiles arrive through the direct-to-LDS ring of
// pkv_ring.h.  The paging follows the flashinfer.cake_fmha API page's contract
// (key j of request b is token j % P of page block_tables[b][j / P]); the
// Split-KV partials (normalized O and natural-log LSE per partition, merged
// by the separate reducer) follow the PR #4557 page's Split-KV description.

#include <cfloat>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_ring.h"

namespace pkv {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int DQK_, int DV_, bool VSHARE_, int RB_, int NW_, int KB_, int NS_, int OCC_ = 1>
struct M32Cfg {
  static constexpr int DQK = DQK_, DV = DV_, RB = RB_, NW = NW_, KB = KB_, NS = NS_;
  static constexpr int OCC = OCC_;  // waves per SIMD the register budget is sized for
  // read-ahead distance (in MFMA steps) of the K and V^T operand reads;
  // shorter for long rows, whose Q and O already fill the register file
  static constexpr int PDK = DQK > 256 ? 3 : 4;
  static constexpr int PDV = DQK > 256 ? 3 : 4;
  static constexpr bool VSHARE = VSHARE_;
  static constexpr int NTHR = 64 * NW;
  static constexpr int ROWS = NW * RB * 32;  // packed query rows per workgroup
  static constexpr int T = KB * 32;          // keys per ring stage
  static constexpr int KROWB = DQK * 2;
  static constexpr int VROWB = VSHARE ? KROWB : DV * 2;
  static constexpr int NCK = KROWB / 16;
  static constexpr int NCV = VROWB / 16;
  static constexpr int KTILE = T * KROWB;
  static constexpr int VTILE = VSHARE ? 0 : T * VROWB;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KCH = T * NCK;
  static constexpr int VCH = VSHARE ? 0 : T * NCV;
  static constexpr int NI = (KCH + VCH) / 64;  // wave-instructions per stage
  static constexpr int KPW = (NI + NW - 1) / NW;
  static constexpr int NKS = DQK / 16;  // 16-wide k steps of S^T
  static constexpr int NDB = DV / 32;  // 32-wide value blocks of O^T per wave
  static constexpr int LDS = NS * STAGE;
  // recompute the loader's per-lane geometry every stage instead of keeping it
  // live: long rows, or more than one wave per SIMD (registers are the limit)
  static constexpr bool LEAN = DQK > 256 || OCC > 1;
  static constexpr bool ROW16 = NCK == 16 && (VSHARE || NCV == 16);  // closed-form loader geometry
  static_assert(KCH % 64 == 0 && VCH % 64 == 0, "wave-instructions must not straddle K and V");
  static_assert(KPW * (NS - 1) < 64, "vmcnt holds at most 63 outstanding loads");
  static_assert(DQK % 16 == 0 && DV % 32 == 0 && NCK % 4 == 0 && NCV % 4 == 0, "tiling");
  static_assert(NS >= 2 && NS <= 6, "ring depth");
  static_assert(!VSHARE || DV <= DQK, "shared V rows");
};

// Swizzle key of LDS row r (K and V rows alike): 16-byte chunk c of the row is
// stored at c ^ (key & group mask).  Chosen for the two read patterns: the
// eight rows {0-3, 8-11} (+4, +16) that one ds_read_b128 serves together get
// eight distinct keys, and the four rows of each 16-lane transpose read get
// chunk pairs that do not overlap.
__device__ __forceinline__ int m32_key(int r) { return 4 * (r & 3) + 2 * ((r >> 3) & 1); }

// Physical chunk of logical chunk c_const + c_lane where c_lane < 4 never leaves
// c_const's swizzle group.  With c_const a compile-time constant only the XOR of
// the low bits depends on the lane, so offsets differing by whole groups fold
// into instruction immediates.
template <int NC>
__device__ __forceinline__ int chunk_phys(int c_const, int c_lane, int key) {
  const int m = swz_mask<NC>(c_const);
  return (c_const & ~m) + (((c_const & m) + c_lane) ^ (key & m));
}

// Compile-time loop: f receives the index as a std::integral_constant
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Registers per wave holding the page list (64 pages each); the planner caps a
// partition of these kernels at 64 * kPageRegs pages
constexpr int kPageRegs = kM32MaxPages / 64;

// Largest rise of a row's max (log2 units) absorbed without rescaling O
constexpr float kLazyMax = 8.f;


// A row r of S^T reads key r with bits 2 and 3 exchanged
__device__ __forceinline__ int m32_perm(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <class C>
__device__ __forceinline__ void m32_block(const KParams& p, unsigned char* smem, int32_t* s_pages, const int b,
                                          const int g, const int rblk, const int part_lo, const int part_hi,
                                          const int slot, const bool lead) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  const int h = lane >> 5;   // k half of the operands, row quad of the results
  const int c32 = lane & 31;  // query row inside a 32-row block
  const int G = p.group;
  const int wr = wave;  // row group of this wave

  __syncthreads();  // LDS of a previous piece is free again (no loads are in flight here)

  int t0, n_b;
  if (p.is_context) {
    int a0 = p.q_indptr[b], a1 = p.q_indptr[b + 1];
    bool bad = (a0 < 0) || (a1 < a0) || (a1 - a0 > p.max_q_len) || (a1 > p.total_q);
    if (bad) {
      if (lead && g == 0 && rblk == 0 && tid == 0) flag_error(p.err_word, PKV_DEVERR_QINDPTR);
      return;
    }
    t0 = a0;
    n_b = a1 - a0;
  } else {
    t0 = b * p.q_len;
    n_b = p.q_len;
  }
  const int row_space = n_b * G;
  const int row0 = rblk * C::ROWS;
  if (row0 >= row_space) return;

  int L = p.seq_lens[b];
  const int cap = p.max_pages_per_seq * p.page_size;
  if (lead && g == 0 && rblk == 0 && tid == 0) {
    if (L > cap) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_TABLE);
    if (L > p.max_kv_len) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_MAXLEN);
    if (L < n_b) flag_error(p.err_word, PKV_DEVERR_SEQ_LT_QLEN);
  }
  L = max(0, min(L, p.kv_span));

  const int last_row = min(row0 + C::ROWS, row_space) - 1;
  const int i_max = last_row / G;
  const int c_max = p.causal ? min(L, max(0, L - n_b + i_max + 1)) : L;
  const int kv_lo = part_lo;
  const int kv_hi = min(part_hi, c_max);
  const int n_tiles = kv_hi > kv_lo ? (kv_hi - kv_lo + C::T - 1) / C::T : 0;
  if (n_tiles == 0 && p.ws_o != nullptr) return;

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

  const float k_scale = p.k_scale_dev ? *p.k_scale_dev : p.k_scale;
  const float v_scale = p.v_scale_dev ? *p.v_scale_dev : p.v_scale;
  const float sc2_raw = p.scale * k_scale * kLog2e;
  // a negative logit scale is folded into Q (an exact bf16 sign flip), so the
  // softmax only ever needs the row max of the raw products
  const float sc2 = fmaxf(fabsf(sc2_raw), FLT_MIN);  // > 0: a masked key's -inf score stays -inf
  const uint32_t q_sign = sc2_raw < 0.f ? 0x80008000u : 0u;

  int row_t[C::RB], row_h[C::RB], row_c[C::RB];
  bool row_ok[C::RB];
  bf16x8 qB[C::RB][C::NKS];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const int R = row0 + (wr * C::RB + rb) * 32 + c32;
    row_ok[rb] = R < row_space;
    const int i = row_ok[rb] ? R / G : 0;
    row_t[rb] = t0 + i;
    row_h[rb] = g * G + (row_ok[rb] ? R % G : 0);
    const int c = p.causal ? L - n_b + i + 1 : L;
    row_c[rb] = row_ok[rb] ? min(max(c, 0), kv_hi) : 0;
    const __bf16* qrow = (const __bf16*)p.q + row_t[rb] * p.q_st + row_h[rb] * p.q_sh + 8 * h;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const bf16x8 q = row_ok[rb] ? *(const bf16x8*)(qrow + 16 * ks) : bf16x8{};
      u32x4 qw = __builtin_bit_cast(u32x4, q);
      qw ^= u32x4{q_sign, q_sign, q_sign, q_sign};
      qB[rb][ks] = __builtin_bit_cast(bf16x8, qw);
    }
  }

  // visible-key bounds over this wave's rows: blocks below c_lo need no mask,
  // blocks at or past c_hi hold no visible key of any of its rows
  int c_lo = INT_MAX, c_hi = 0;
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb)
    if (row_ok[rb]) {
      c_lo = min(c_lo, row_c[rb]);
      c_hi = max(c_hi, row_c[rb]);
    }
  c_lo = __builtin_amdgcn_readfirstlane(-wave_max_i(-c_lo));  // wave-uniform: scalar branches below
  c_hi = __builtin_amdgcn_readfirstlane(wave_max_i(c_hi));

  // Row sums: each lane sums its weights of a block in fp32 (l_run); the two
  // lanes of a row are added at the end.
  float m_run[C::RB], l_run[C::RB];
  f32x16 O[C::RB][C::NDB];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) O[rb][d][e] = 0.f;
  }

  __syncthreads();  // page list visible

  // The validated page list also sits in registers, lane l of pl[k] holding
  // page 64k + l (the planner keeps a partition within 64 * kPageRegs pages): a
  // wave-instruction's page is then one v_readlane, with no memory access whose
  // wait counter would also cover the ring's loads in flight.
  int pl[kPageRegs], plv[kPageRegs];  // K pages, V pages (the same list without a V table)
#pragma unroll
  for (int k = 0; k < kPageRegs; ++k) {
    pl[k] = 64 * k + lane < n_pg ? s_pages[64 * k + lane] : 0;
    plv[k] = 64 * k + lane < n_pg ? s_vpages[64 * k + lane] : 0;
  }
  auto page_of = [&](int idx, bool is_k) -> uint32_t {
    int v = __builtin_amdgcn_readlane(is_k ? pl[0] : plv[0], idx & 63);
#pragma unroll
    for (int k = 1; k < kPageRegs; ++k)
      if ((idx >> 6) == k) v = __builtin_amdgcn_readlane(is_k ? pl[k] : plv[k], idx & 63);
    return (uint32_t)v;
  };

  // ---- loader: wave-instruction q of this wave fills chunks I*64 .. I*64+63 of the
  // stage (I = wave*KPW + q); lane l fetches the global chunk whose swizzled LDS slot
  // is I*64 + l.
  const int pmask = p.page_size - 1;
  const uint32_t k_tok_b = (uint32_t)(p.k_stok * 2), v_tok_b = (uint32_t)(p.v_stok * 2);
  const uint32_t k_head_b = (uint32_t)(g * p.k_sh * 2), v_head_b = (uint32_t)(g * p.v_sh * 2);
  const uint64_t k_pg_b = (uint64_t)p.k_sp * 2, v_pg_b = (uint64_t)p.v_sp * 2;
  const uint64_t k_addr = (uint64_t)p.k, v_addr = (uint64_t)p.v;
  auto geometry = [&](int ln, int* q_row, uint32_t* q_chunk) {
#pragma unroll
    for (int q = 0; q < C::KPW; ++q) {
      const int I = min(wave * C::KPW + q, C::NI - 1);
      const int P = I * 64 + ln;
      if (I * 64 < C::KCH) {
        const int r = P / C::NCK, ph = P % C::NCK;
        q_row[q] = r;
        q_chunk[q] = (uint32_t)((ph ^ (m32_key(r) & swz_mask<C::NCK>(ph))) * 16);
      } else {
        const int Pv = P - C::KCH;
        const int r = Pv / C::NCV, ph = Pv % C::NCV;
        q_row[q] = r;
        q_chunk[q] = (uint32_t)((ph ^ (m32_key(r) & swz_mask<C::NCV>(ph))) * 16);
      }
    }
  };
  int g_row[C::LEAN ? 1 : C::KPW];
  uint32_t g_chunk[C::LEAN ? 1 : C::KPW];
  if constexpr (!C::LEAN && !C::ROW16) geometry(lane, g_row, g_chunk);
  // 16-chunk rows (D = 128, bf16): wave-instruction I' of a tile (counted
  // within the K or the V part) fills rows 4I' .. 4I'+3, lane l taking row
  // 4I' + l/16 and physical chunk l%16; the swizzle key of that row is
  // 4(l/16) + 2((I'/2)%2), so the logical chunk is a lane constant XOR a
  // uniform bit and no per-lane geometry needs to be stored or recomputed.
  const int g16_row = lane >> 4;
  const uint32_t g16_chunk = (uint32_t)((lane & 15) ^ (4 * (lane >> 4)));
  // Every wave-instruction covers consecutive rows of one page (the planner
  // guarantees it: rows per instruction divide the page, or the whole tile sits
  // in one page), so its page base is wave-uniform: looked up once, added on
  // the scalar unit, and each lane only supplies its 32-bit in-page offset.
  auto issue = [&](int tile, int stage, int q_lo = 0, int q_hi = C::KPW) {
    const int tok0 = kv_lo + tile * C::T;
    unsigned char* st = smem + stage * C::STAGE;
    int q_row_l[C::KPW];
    uint32_t q_chunk_l[C::KPW];
    const int* q_row = q_row_l;
    const uint32_t* q_chunk = q_chunk_l;
    if constexpr (C::ROW16) {
#pragma unroll
      for (int q = 0; q < C::KPW; ++q) {
        const int I = min(wave * C::KPW + q, C::NI - 1);
        const int Ip = I * 64 < C::KCH ? I : I - C::KCH / 64;
        q_row_l[q] = 4 * Ip + g16_row;
        q_chunk_l[q] = (g16_chunk ^ (uint32_t)(2 * ((Ip >> 1) & 1))) * 16;
      }
    } else if constexpr (C::LEAN) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      geometry(ln, q_row_l, q_chunk_l);
    } else {
      q_row = g_row;
      q_chunk = g_chunk;
    }
    uint32_t pgv[C::KPW];
#pragma unroll
    for (int q = 0; q < C::KPW; ++q) {
      if (q < q_lo || q >= q_hi) continue;
      const int I = min(wave * C::KPW + q, C::NI - 1);
      const int r0 = I * 64 < C::KCH ? (I * 64) / C::NCK : (I * 64 - C::KCH) / C::NCV;
      const int tokf = __builtin_amdgcn_readfirstlane(min(tok0 + r0, kv_hi - 1));
      pgv[q] = page_of((tokf >> p.log2_page) - pg_lo, I * 64 < C::KCH);
    }
#pragma unroll
    for (int q = 0; q < C::KPW; ++q) {
      if (q < q_lo || q >= q_hi) continue;
      const int I = min(wave * C::KPW + q, C::NI - 1);
      const bool is_k = I * 64 < C::KCH;
      const uint32_t pg = pgv[q];
      const uint64_t sbase = (is_k ? k_addr + k_head_b : v_addr + v_head_b) + (uint64_t)pg * (is_k ? k_pg_b : v_pg_b);
      const int tok = min(tok0 + q_row[q], kv_hi - 1);
      const uint32_t voff = (uint32_t)(tok & pmask) * (is_k ? k_tok_b : v_tok_b) + q_chunk[q];
      dma16_saddr(sbase, voff, st + I * 1024);
    }
  };

  // ---- per-lane operand offsets inside a stage (constant parts fold into immediates)
  const int kkey = m32_perm(c32);  // key read by A row c32 of S^T, inside each 32-key block
  const int kfk = m32_key(kkey);
  const int kl_row = kkey * C::KROWB;
  // V^T transpose reads: 16-lane group q = lane/16 covers values 16(q&1) .. +15 and
  // keys 8(q>>1) + 4*half + (lane%16)/4; source lane j = lane%16 supplies 4 values
  // of one key row at value offset 4(j%4)
  const int vj = lane & 15;
  const int vq = lane >> 4;
  const int vrow = 8 * (vq >> 1) + (vj >> 2);
  const int vfk = m32_key(vrow);
  const int vc_lane = 2 * (vq & 1) + ((vj & 3) >> 1);
  const int vl_row = vrow * C::VROWB + 8 * (vj & 1);

  // ---- the pieces of one 32-key block
  // Online softmax (exp2 domain); element e of acc holds key 16(e/8) + 8h + e%8.
  // The running max only moves when a score exceeds it by more than kLazyMax
  // (log2 units): below that the stale max keeps every weight within
  // 2^kLazyMax, and since the sum and O share that reference the result is
  // unchanged -- O is rescaled only on real jumps.
  auto softmax = [&](int j, const f32x16 (&acc)[C::RB], bf16x8 (&pb)[C::RB][2]) {
    const int blk_tok = kv_lo + j * 32;
    const bool full = blk_tok + 32 <= c_lo;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      float w[16];
      float mx;
      if (full) {
        // scores are acc * sc2 with sc2 >= 0: reduce the raw accumulators, scale once
        float mr = acc[rb][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mr = fmaxf(mr, acc[rb][e]);
        mx = half_swap_max(mr) * sc2;
      } else {
        mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int tok = blk_tok + 16 * (e >> 3) + 8 * h + (e & 7);
          w[e] = tok < row_c[rb] ? acc[rb][e] * sc2 : -INFINITY;
          mx = fmaxf(mx, w[e]);
        }
        mx = half_swap_max(mx);
      }
      const bool move = mx > m_run[rb] + kLazyMax;  // also true on a row's first visible key
      const float m_new = move ? mx : m_run[rb];
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = move ? fast_exp2(m_run[rb] - m_use) : 1.f;
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) O[rb][d] *= alpha;
      }
      m_run[rb] = m_new;
      if (full) {
#pragma unroll
        for (int e = 0; e < 16; ++e) w[e] = fast_exp2(fmaf(acc[rb][e], sc2, -m_use));
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) w[e] = fast_exp2(w[e] - m_use);
      }
      float ls = w[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) ls += w[e];
      l_run[rb] = fmaf(l_run[rb], alpha, ls);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 wv{pack_bf16x2(w[8 * st + 0], w[8 * st + 1]), pack_bf16x2(w[8 * st + 2], w[8 * st + 3]),
                 pack_bf16x2(w[8 * st + 4], w[8 * st + 5]), pack_bf16x2(w[8 * st + 6], w[8 * st + 7])};
        pb[rb][st] = __builtin_bit_cast(bf16x8, wv);
      }
    }
  };
  // Products with their LDS operand reads interleaved: a ring of PD operands
  // in registers, each read issued PD MFMA steps before the MFMA that uses it
  // (registers stay at PD operands instead of a whole block's worth).
  auto s_product_ring = [&](int j, f32x16 (&acc)[C::RB]) {
    const unsigned char* kblk = smem + ((j / C::KB) % C::NS) * C::STAGE + (j % C::KB) * 32 * C::KROWB + kl_row;
    auto rd = [&](int ks) { return *(const bf16x8*)(kblk + chunk_phys<C::NCK>(2 * ks, h, kfk) * 16); };
    constexpr int PD = C::PDK < C::NKS ? C::PDK : C::NKS;
    bf16x8 ring[PD];
#pragma unroll
    for (int q = 0; q < PD; ++q) ring[q] = rd(q);
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[rb][e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      const bf16x8 a = ring[ks % PD];
      if (ks + PD < C::NKS) ring[ks % PD] = rd(ks + PD);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) acc[rb] = mfma32x32x16(a, qB[rb][ks], acc[rb]);
    }
  };
  auto pv_product_ring = [&](int j, const bf16x8 (&pb)[C::RB][2]) {
    const unsigned char* vst = smem + ((j / C::KB) % C::NS) * C::STAGE + (C::VSHARE ? 0 : C::KTILE);
    const unsigned char* vblk = vst + (j % C::KB) * 32 * C::VROWB + vl_row;
    auto rd = [&](int i) {  // i = 2 db + st
      const int db = i >> 1, st = i & 1;
      const unsigned char* src = vblk + 16 * st * C::VROWB + chunk_phys<C::NCV>(4 * db, vc_lane, vfk) * 16;
      const s16x4 lo = lds_read_tr16(src);
      const s16x4 hi = lds_read_tr16(src + 4 * C::VROWB);
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      return __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    constexpr int N = 2 * C::NDB;
    constexpr int PD = C::PDV < N ? C::PDV : N;
    bf16x8 ring[PD];
#pragma unroll
    for (int q = 0; q < PD; ++q) ring[q] = rd(q);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bf16x8 a = ring[i % PD];
      if (i + PD < N) ring[i % PD] = rd(i + PD);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) O[rb][i >> 1] = mfma32x32x16(a, pb[rb][i & 1], O[rb][i >> 1]);
    }
  };
  // PV product of block jP with the softmax of block jS (whose S^T product
  // just ended) in pieces between its MFMAs: the wave's own vector work then
  // runs in the shadow of its matrix work instead of only beside the other
  // wave of the SIMD.  Each piece ties its results to an empty asm statement
  // so that it stays between the MFMAs around it.  The rescale of O for block
  // jS (rare) follows the last MFMA of block jP.
  float sm_mx[C::RB], sm_use[C::RB], sm_alpha[C::RB], sm_ls[C::RB];
  bool sm_move[C::RB];
  auto softmax_piece = [&](auto piece, int jS, f32x16 (&acc)[C::RB], bf16x8 (&pb)[C::RB][2]) {
    constexpr int c = decltype(piece)::value;
    const int blk_tok = kv_lo + jS * 32;
    const bool full = blk_tok + 32 <= c_lo;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      if constexpr (c == 0) {
        if (!full) {  // keys at or past the row's causal limit weigh zero (sc2 > 0)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (blk_tok + 16 * (e >> 3) + 8 * h + (e & 7) >= row_c[rb]) acc[rb][e] = -INFINITY;
        }
        float mx = acc[rb][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, acc[rb][e]);
        sm_mx[rb] = mx;
        asm volatile("" : "+v"(sm_mx[rb]));
      } else if constexpr (c == 1) {
#pragma unroll
        for (int e = 8; e < 16; ++e) sm_mx[rb] = fmaxf(sm_mx[rb], acc[rb][e]);
        asm volatile("" : "+v"(sm_mx[rb]));
      } else if constexpr (c == 2) {
        const float mx = half_swap_max(sm_mx[rb]) * sc2;
        sm_move[rb] = mx > m_run[rb] + kLazyMax;  // also true on a row's first visible key
        const float m_new = sm_move[rb] ? mx : m_run[rb];
        sm_use[rb] = (m_new == -INFINITY) ? 0.f : m_new;
        sm_alpha[rb] = sm_move[rb] ? fast_exp2(m_run[rb] - sm_use[rb]) : 1.f;
        m_run[rb] = m_new;
        sm_ls[rb] = 0.f;
        asm volatile("" : "+v"(sm_use[rb]), "+v"(sm_alpha[rb]), "+v"(m_run[rb]));
      } else if constexpr (c < 19) {
        constexpr int e = c - 3;
        acc[rb][e] = fast_exp2(fmaf(acc[rb][e], sc2, -sm_use[rb]));
        sm_ls[rb] += acc[rb][e];
        asm volatile("" : "+v"(acc[rb][e]), "+v"(sm_ls[rb]));
      } else {
        l_run[rb] = fmaf(l_run[rb], sm_alpha[rb], sm_ls[rb]);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          u32x4 wv{pack_bf16x2(acc[rb][8 * st + 0], acc[rb][8 * st + 1]),
                   pack_bf16x2(acc[rb][8 * st + 2], acc[rb][8 * st + 3]),
                   pack_bf16x2(acc[rb][8 * st + 4], acc[rb][8 * st + 5]),
                   pack_bf16x2(acc[rb][8 * st + 6], acc[rb][8 * st + 7])};
          pb[rb][st] = __builtin_bit_cast(bf16x8, wv);
        }
        asm volatile("" : "+v"(pb[rb][0]), "+v"(pb[rb][1]), "+v"(l_run[rb]));
      }
    }
  };
  constexpr int kPieces = 20;
  auto pv_softmax = [&](int jP, const bf16x8 (&pbP)[C::RB][2], int jS, f32x16 (&acc)[C::RB],
                        bf16x8 (&pbS)[C::RB][2]) {
    const unsigned char* vst = smem + ((jP / C::KB) % C::NS) * C::STAGE + (C::VSHARE ? 0 : C::KTILE);
    const unsigned char* vblk = vst + (jP % C::KB) * 32 * C::VROWB + vl_row;
    auto rd = [&](int i) {  // i = 2 db + st
      const int db = i >> 1, st = i & 1;
      const unsigned char* src = vblk + 16 * st * C::VROWB + chunk_phys<C::NCV>(4 * db, vc_lane, vfk) * 16;
      const s16x4 lo = lds_read_tr16(src);
      const s16x4 hi = lds_read_tr16(src + 4 * C::VROWB);
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      return __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
    constexpr int N = 2 * C::NDB;
    constexpr int PD = C::PDV < N ? C::PDV : N;
    bf16x8 ring[PD];
#pragma unroll
    for (int q = 0; q < PD; ++q) ring[q] = rd(q);
    static_for<0, N>([&](auto slot) {
      constexpr int i = decltype(slot)::value;
      const bf16x8 a = ring[i % PD];
      if (i + PD < N) ring[i % PD] = rd(i + PD);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) O[rb][i >> 1] = mfma32x32x16(a, pbP[rb][i & 1], O[rb][i >> 1]);
      static_for<0, kPieces>([&](auto piece) {
        constexpr int c = decltype(piece)::value;
        if constexpr ((c * N) / kPieces == i) softmax_piece(piece, jS, acc, pbS);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      if (__builtin_amdgcn_ballot_w64(sm_move[rb]) != 0) {
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) O[rb][d] *= sm_alpha[rb];
      }
    }
  };
  // Start of ring tile t: this wave's loads of t are complete once at most
  // (tiles issued after t) * KPW remain; the barrier then publishes every wave's
  // part and frees the stage of tile t-1, which the next issue refills.
  auto tile_start = [&](int t, bool issue_now = true) {
    const int after = min(C::NS - 2, n_tiles - 1 - t);
    if constexpr (C::NS >= 5) {
      if (after >= 3) wait_loads<3 * C::KPW>();
      else if (after == 2) wait_loads<2 * C::KPW>();
      else if (after == 1) wait_loads<C::KPW>();
      else wait_loads<0>();
    } else if constexpr (C::NS == 4) {
      if (after >= 2) wait_loads<2 * C::KPW>();
      else if (after == 1) wait_loads<C::KPW>();
      else wait_loads<0>();
    } else if constexpr (C::NS == 3) {
      if (after >= 1) wait_loads<C::KPW>();
      else wait_loads<0>();
    } else {
      wait_loads<0>();
    }
    ring_barrier();
    if (issue_now && t + C::NS - 1 < n_tiles) issue(t + C::NS - 1, (t + C::NS - 1) % C::NS);
  };

  // prologue: the first NS-1 tiles in flight
#pragma unroll
  for (int t = 0; t < C::NS - 1; ++t)
    if (t < n_tiles) issue(t, t);

  // 32-key blocks: S^T product (K operands read a few MFMA steps ahead),
  // softmax, PV product, with the softmax of block j in the shadow of the PV
  // product of block j-1 inside a tile.  The two waves of a SIMD also run
  // independently between the tile barriers, so one's matrix work covers the
  // other's vector work.  Blocks past this wave's last visible key are
  // skipped; every wave still takes every tile's barrier.
  f32x16 accA[C::RB];
  auto active = [&](int j) { return kv_lo + j * 32 < c_hi; };
  // Within a tile: S^T(j), then PV(j-1) with the softmax of block j in its
  // shadow; the tile's first softmax runs alone and its last PV product
  // before the next tile's barrier, which frees the stage for a refill.
  for (int t = 0; t < n_tiles; ++t) {
    tile_start(t);
    const int j0 = t * C::KB;
    if (!active(j0)) continue;
    bf16x8 pb_cur[C::RB][2], pb_prev[C::RB][2];
    s_product_ring(j0, accA);
    softmax(j0, accA, pb_cur);
    int j = j0;
    for (int k = 1; k < C::KB; ++k) {
      if (!active(j0 + k)) break;
      j = j0 + k;
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
        pb_prev[rb][0] = pb_cur[rb][0];
        pb_prev[rb][1] = pb_cur[rb][1];
      }
      s_product_ring(j, accA);
      pv_softmax(j - 1, pb_prev, j, accA, pb_cur);
    }
    pv_product_ring(j, pb_cur);
  }

  // ---- full row sums
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) l_run[rb] = half_swap_sum(l_run[rb]);

  // ---- epilogue: element e of O[rb][db] is value 32db + 8(e/4) + 4h + e%4 of row c32
  const bool split_mode = p.ws_o != nullptr;
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    if (!row_ok[rb]) continue;
    const bool empty = !(l_run[rb] > 0.f);
    float inv = empty ? 0.f : v_scale / l_run[rb];
    float lse = empty ? -INFINITY : (m_run[rb] * kLn2 + __logf(l_run[rb]));
    if (p.sinks && !split_mode) inv *= fold_sink(lse, p.sinks[row_h[rb]]);  // split: the reducer adds it
    const int64_t row_g = (int64_t)row_t[rb] * p.num_qo_heads + row_h[rb];
    if (split_mode) {
      const int64_t prow = (int64_t)slot * p.rows_total + row_g;
      if (h == 0) p.ws_lse[prow] = lse;
      if (!empty) {
        float* dst = p.ws_o + prow * C::DV + 4 * h;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(f32x4*)(dst + 32 * d + 8 * q) =
                f32x4{O[rb][d][4 * q], O[rb][d][4 * q + 1], O[rb][d][4 * q + 2], O[rb][d][4 * q + 3]} * inv;
      }
    } else {
      if (p.lse_out && h == 0) p.lse_out[row_g] = lse;
      if (p.o_dtype == PKV_DTYPE_BF16) {
        __bf16* dst = (__bf16*)p.out + row_t[rb] * p.o_st + row_h[rb] * p.o_sh + 4 * h;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x2 w{pack_bf16x2(O[rb][d][4 * q] * inv, O[rb][d][4 * q + 1] * inv),
                    pack_bf16x2(O[rb][d][4 * q + 2] * inv, O[rb][d][4 * q + 3] * inv)};
            *(u32x2*)(dst + 32 * d + 8 * q) = w;
          }
      } else {
        float* dst = (float*)p.out + row_t[rb] * p.o_st + row_h[rb] * p.o_sh + 4 * h;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(f32x4*)(dst + 32 * d + 8 * q) =
                f32x4{O[rb][d][4 * q], O[rb][d][4 * q + 1], O[rb][d][4 * q + 2], O[rb][d][4 * q + 3]} * inv;
      }
    }
  }
}

// Workgroup order.  The hardware hands workgroup i to XCD i % 8 and each XCD has
// its own L2, so consecutive logical work items (the row blocks of one request
// and KV head, which read the same pages) are placed on one XCD.  For causal
// context the row blocks are also taken heaviest first (later query positions
// see more keys), so that every CU receives a mix of long and short blocks.
template <class C>
__global__ __launch_bounds__(C::NTHR, C::OCC) void attn_m32_kernel(const KParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pages = (int32_t*)(smem + C::LDS);
  const int nx = gridDim.x, ny = gridDim.y, nz = gridDim.z;
  const int rbc = p.row_blocks;
  const int64_t N = (int64_t)nx * ny * nz;
  const int64_t P = blockIdx.x + (int64_t)nx * (blockIdx.y + (int64_t)ny * blockIdx.z);
  int split, y, z;
  const int64_t per = N / 8;
  if (N % 8 == 0 && nx == 1 && p.is_context && p.causal && per % rbc == 0) {
    const int64_t groups = per / rbc;  // (request, KV head) groups per XCD
    const int64_t xcd = P % 8, idx = P / 8;
    const int rb = rbc - 1 - (int)(idx / groups);
    const int64_t grp = xcd * groups + idx % groups;  // = b * Hkv + g
    split = 0;
    z = (int)(grp / p.num_kv_heads);
    y = (int)(grp % p.num_kv_heads) * rbc + rb;
  } else {
    const int64_t Lg = N % 8 == 0 ? (P % 8) * per + P / 8 : P;
    split = (int)(Lg % nx);
    y = (int)((Lg / nx) % ny);
    z = (int)(Lg / ((int64_t)nx * ny));
  }
  const int span = p.pages_per_split * p.page_size;
  m32_block<C>(p, smem, s_pages, z, y / rbc, y % rbc, split * span, split * span + span, split, split == 0);
}

// ---------------------------------------------------------------- instances
//                          DQK  DV   VSH    RB NW KB NS OCC
// 256 rows on 8 waves (two per SIMD), two 64 KiB stages of 128 keys
using M32CtxW8T128 = M32Cfg<128, 128, false, 1, 8, 4, 2, 2>;

template <class C>
static void fill_m32_shape(MfmaShape* s) {
  s->rows_per_block = C::ROWS;
  s->tile_tokens = C::T;
  s->threads = C::NTHR;
  s->lds_static = C::LDS;
}

bool m32_shape(int32_t kernel, MfmaShape* s) {
  if (kernel != KERNEL_M32_CTX_W8T128) return false;
  fill_m32_shape<M32CtxW8T128>(s);
  return true;
}

template <class C>
static hipError_t launch_m32_cfg(const KParams& p, hipStream_t s) {
  static bool attr_done = false;  // idempotent; a race only repeats the same call
  const size_t list = (size_t)p.page_list_cap * (p.v_table ? 2 : 1);
  const size_t lds = C::LDS + ((list + 3) & ~size_t(3)) * sizeof(int32_t);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_m32_kernel<C>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  dim3 grid(p.num_splits, p.num_kv_heads * p.row_blocks, p.batch);
  hipLaunchKernelGGL(attn_m32_kernel<C>, grid, dim3(C::NTHR), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_m32(int32_t kernel, const KParams& p, hipStream_t s) {
  if (kernel == KERNEL_M32_CTX_W8T128) return launch_m32_cfg<M32CtxW8T128>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv

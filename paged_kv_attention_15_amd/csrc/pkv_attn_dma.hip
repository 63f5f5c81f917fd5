// pkv_attn_dma.hip -- MFMA paged attention fed by a multi-stage direct-to-LDS ring.
//
// Same contract and tile mathematics as pkv_attn_mfma.hip (S^T = K Q^T, online
// softmax in the exp2 domain, O^T += V^T P^T on v_mfma_f32_16x16x32_bf16), with
// a different loader:
//   * the block-table gather issues global_load_lds_dwordx4 (16 bytes per lane,
//     straight into LDS, no staging registers).  Lane l of one wave-instruction
//     lands at (LDS base + 16*l), so the chunk XOR swizzle is applied by
//     choosing which global chunk each lane fetches;
//   * NS LDS stages form a ring: NS-1 tiles are in flight while one is
//     computed, and each wave waits (s_waitcnt vmcnt) only for the tile it is
//     about to read; a plain s_barrier (no fence, so no forced drain of the
//     ring) then publishes every wave's part of that tile;
//   * K and V stay in their stored dtype in LDS (e4m3 halves the LDS per key
//     and doubles the keys in flight) and are converted to bf16 when they are
//     read into MFMA operands: K rows with ds_read_b64 + v_cvt_scalef32_pk_bf16_fp8,
//     V^T with ds_read_b64_tr_b8 (8 keys of one channel per lane) for e4m3 or
//     two ds_read_b64_tr_b16 for bf16;
//   * within each 32-key chunk the K rows fed to the MFMA A operand are
//     permuted (A row r of sub-block h takes key 8*(r/4) + 4*h + r%4) so that
//     the 16-lane group G of the S^T result holds keys 8G..8G+7 -- the same
//     eight consecutive keys the transpose reads deliver for V^T -- and P^T
//     feeds the PV product without any cross-lane movement.
// The paging itself follows the flashinfer.cake_fmha API page's contract (key j
// of request b is token j % P of page block_tables[b][j / P]); Split-KV
// partials and the balanced schedule are those of pkv_attn_mfma.hip.

#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_ring.h"

namespace pkv {

template <int DQK_, int DV_, bool FP8_, bool VSHARE_, int RT_, int NWR_, int NWT_, int TT_, int NS_>
struct DmaCfg {
  static constexpr int DQK = DQK_, DV = DV_, RT = RT_, NWR = NWR_, NWT = NWT_, TT = TT_, NS = NS_;
  static constexpr bool FP8 = FP8_, VSHARE = VSHARE_;
  static constexpr int NW = NWR * NWT;
  static constexpr int NTHR = 64 * NW;
  static constexpr int T = NWT * TT;
  static constexpr int ROWS = NWR * RT * 16;
  static constexpr int EB = FP8 ? 1 : 2;
  static constexpr int KROWB = DQK * EB;                 // LDS bytes per K row (stored dtype)
  static constexpr int VROWB = VSHARE ? KROWB : DV * EB;
  static constexpr int NCK = KROWB / 16;                 // 16-byte chunks per row
  static constexpr int NCV = VROWB / 16;
  static constexpr int KTILE = T * KROWB;
  static constexpr int VTILE = VSHARE ? 0 : T * VROWB;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KCH = T * NCK;
  static constexpr int VCH = VSHARE ? 0 : T * NCV;
  static constexpr int NI = (KCH + VCH) / 64;            // wave-instructions per tile
  // per wave; when NI is not a multiple of NW the last instruction is repeated
  // (same source, same destination: an idempotent reload) so that every wave
  // issues the same count and the vmcnt bookkeeping stays uniform
  static constexpr int KPW = (NI + NW - 1) / NW;
  static constexpr int NKS = DQK / 32;
  static constexpr int NDB = DV / 16;
  static constexpr int NNB = TT / 16;
  static constexpr int RED_O = NWT > 1 ? NW * RT * NDB * 64 * 16 : 0;
  static constexpr int RED_ML = NWT > 1 ? NW * RT * 64 * 2 * 4 : 0;
  static constexpr int LDS = (NS * STAGE > RED_O + RED_ML) ? NS * STAGE : RED_O + RED_ML;
  static_assert(KCH % 64 == 0 && VCH % 64 == 0, "wave-instructions must not straddle K and V");
  static_assert(KPW * (NS - 1) < 64, "vmcnt holds at most 63 outstanding loads");
  static_assert(TT % 32 == 0 && DQK % 32 == 0 && DV % 16 == 0, "MFMA tiling");
  static_assert(NS >= 2 && NS <= 6, "ring depth");
  // very long rows (MLA): registers are the limit, so per-lane addresses are
  // recomputed every tile instead of being kept live (cheap VALU vs. spills)
  static constexpr bool LEAN = DQK > 256;
  static_assert(!VSHARE || DV <= DQK, "shared V rows");
  // bf16 operand reads split the swizzle per step group (phys_chunk_split): K rows
  // hold exactly the chunks the S^T loop walks, V rows at least those of the PV loop
  static_assert(FP8 || (NCK == 4 * NKS && NCV >= 2 * NDB), "operand chunk walk");
};

// Swizzle keys.  K rows are read 16 at a time in the permuted order
// {0-3, 8-11, 16-19, 24-27} (+4): key (r & 3) | ((r >> 1) & 12) gives those 16
// rows 16 distinct keys.  Separate V buffers are read as runs of consecutive
// rows by the transpose reads: key r & 15.
__device__ __forceinline__ int key_k(int r) { return (r & 3) | ((r >> 1) & 12); }

// Largest rise of a row's running max (log2 units) absorbed without rescaling
// O: below it the stale max keeps every weight under 2^kRingLazyMax, and since
// the row sum and O share that reference the result is the same up to rounding.
constexpr float kRingLazyMax = 8.f;
__device__ __forceinline__ int key_v(int r) { return r & 15; }

template <int NC>
__device__ __forceinline__ int phys_chunk(int c, int key) {
  return c ^ (key & swz_mask<NC>(c));
}

// The same chunk for c = base + sub, base a multiple of STEP (4 or 2), sub < STEP
// and base + STEP - 1 < NC.  Then the group mask m of c is that of base and is
// at least STEP - 1, so the XOR only touches the low bits of base:
//   c ^ (key & m) = (base & ~m) + ((base & m) ^ ((sub ^ key) & m)).
// With base an unrolled constant the first term is an immediate, and the
// second takes only a few values per lane (shared between loop steps).
template <int NC, int STEP>
__device__ __forceinline__ int phys_chunk_split(int base, int sub, int key) {
  const int m = swz_mask<NC>(base);
  return (base & ~m) + ((base & m) ^ ((sub ^ key) & m));
}

// Device-coherent word access (agent scope, relaxed): the value goes to or
// comes from the device-wide coherence point rather than one XCD's L2.
__device__ __forceinline__ void st_coherent(float* ptr, float v) {
  __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* ptr) {
  return __hip_atomic_load(const_cast<float*>(ptr), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// VT: the call has a separate V page table (a second page list after the K
// list).  A template parameter rather than a test of p.v_table: the list
// choice in the loader otherwise costs scalar registers the shared-table form
// spills (about 3 % of the e4m3 decode).
template <class C, bool VT = false>
__device__ __forceinline__ void dma_block(const KParams& p, unsigned char* smem, int32_t* s_pages, const int b,
                                          const int g, const int rb, const int part_lo, const int part_hi,
                                          const int slot, const bool lead, const bool direct = false) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches below
  const int wr = wave / C::NWT;
  const int wt = wave % C::NWT;
  const int tid = threadIdx.x;
  const int G4_in = lane >> 4;
  const int l16_in = lane & 15;
  const int G = p.group;

  __syncthreads();  // LDS of a previous piece is free again (no loads are in flight here)

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
  if (row0 >= row_space) return;

  int L = p.seq_lens[b];
  const int cap = p.max_pages_per_seq * p.page_size;
  if (lead && g == 0 && rb == 0 && tid == 0) {
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
  // partial rows go to the workspace unless this piece is the whole key range of its rows
  const bool split_mode = p.ws_o != nullptr && !direct;
  if (n_tiles == 0 && split_mode) return;

  const int pg_lo = kv_lo >> p.log2_page;
  const int n_pg = n_tiles > 0 ? ((kv_hi - 1) >> p.log2_page) - pg_lo + 1 : 0;
  // a separate V table (API page, separate K/V page tables) gets its own list
  // right after the K list
  int32_t* s_vpages = VT ? s_pages + p.page_list_cap : s_pages;
  for (int i = tid; i < n_pg; i += C::NTHR) {
    int pg = p.table[(int64_t)b * p.table_stride + pg_lo + i];
    if (p.num_pages > 0 && (pg < 0 || pg >= p.num_pages)) {
      flag_error(p.err_word, PKV_DEVERR_PAGE_RANGE);
      pg = min(max(pg, 0), p.num_pages - 1);
    }
    s_pages[i] = pg;
    if constexpr (VT) {
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
  const float sc2 = p.scale * k_scale * kLog2e;

  int row_t[C::RT], row_h[C::RT], row_c[C::RT], row_R[C::RT];
  bool row_ok[C::RT];
  bf16x8 qB[C::RT][C::NKS];
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    const int R = row0 + (wr * C::RT + rt) * 16 + l16_in;
    row_R[rt] = R;
    row_ok[rt] = R < row_space;
    const int i = row_ok[rt] ? R / G : 0;
    row_t[rt] = t0 + i;
    row_h[rt] = g * G + (row_ok[rt] ? R % G : 0);
    int c = p.causal ? L - n_b + i + 1 : L;
    row_c[rt] = row_ok[rt] ? min(max(c, 0), kv_hi) : 0;
    const __bf16* qrow = (const __bf16*)p.q + row_t[rt] * p.q_st + row_h[rt] * p.q_sh;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks)
      qB[rt][ks] = row_ok[rt] ? *(const bf16x8*)(qrow + ks * 32 + G4_in * 8) : bf16x8{};
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

  const int pmask = p.page_size - 1;
  // Loader.  Wave-instruction q of this wave fills the 16-byte chunks
  // I*64 .. I*64+63 of the stage (I = wave*KPW + q): lane l fetches the global
  // chunk whose swizzled LDS slot is I*64 + l.  Row and chunk are recomputed
  // for each tile from an opaque lane index (cheaper than keeping them live).
  // In-page offsets fit 32 bits; the page term is one 64-bit multiply-add.
  const uint32_t k_tok_b = (uint32_t)(p.k_stok * C::EB), v_tok_b = (uint32_t)(p.v_stok * C::EB);
  const uint32_t k_head_b = (uint32_t)(g * p.k_sh * C::EB), v_head_b = (uint32_t)(g * p.v_sh * C::EB);
  const uint64_t k_pg_b = (uint64_t)p.k_sp * C::EB, v_pg_b = (uint64_t)p.v_sp * C::EB;
  const uint64_t k_addr = (uint64_t)p.k, v_addr = (uint64_t)p.v;
  auto geometry = [&](int ln, int* q_row, uint32_t* q_chunk) {
#pragma unroll
    for (int q = 0; q < C::KPW; ++q) {
      const int I = min(wave * C::KPW + q, C::NI - 1);
      // non-negative: unsigned division by the (not power-of-two) chunk count
      const uint32_t P = (uint32_t)I * 64u + (uint32_t)ln;
      if (I * 64 < C::KCH) {
        const int r = (int)(P / C::NCK), ph = (int)(P % C::NCK);
        q_row[q] = r;
        q_chunk[q] = (uint32_t)((ph ^ (key_k(r) & swz_mask<C::NCK>(ph))) * 16);
      } else {
        const uint32_t Pv = P - C::KCH;
        const int r = (int)(Pv / C::NCV), ph = (int)(Pv % C::NCV);
        q_row[q] = r;
        q_chunk[q] = (uint32_t)((ph ^ (key_v(r) & swz_mask<C::NCV>(ph))) * 16);
      }
    }
  };
  int g_row[C::LEAN ? 1 : C::KPW];
  uint32_t g_chunk[C::LEAN ? 1 : C::KPW];
  if constexpr (!C::LEAN) geometry(lane, g_row, g_chunk);
  auto issue = [&](int tile, int stage) {
    const int tok0 = kv_lo + tile * C::T;
    unsigned char* st = smem + stage * C::STAGE;
    int q_row_l[C::KPW];
    uint32_t q_chunk_l[C::KPW];
    const int* q_row = q_row_l;
    const uint32_t* q_chunk = q_chunk_l;
    if constexpr (C::LEAN) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      ln &= 63;  // the lane range, hidden by the asm statement
      geometry(ln, q_row_l, q_chunk_l);
    } else {
      q_row = g_row;
      q_chunk = g_chunk;
    }
    int pg[C::KPW];
#pragma unroll
    for (int q = 0; q < C::KPW; ++q) {
      const int I = min(wave * C::KPW + q, C::NI - 1);
      const int tok = min(tok0 + q_row[q], kv_hi - 1);
      const int32_t* list = (VT && I * 64 >= C::KCH) ? s_vpages : s_pages;  // wave-uniform: K or V chunks
      pg[q] = list[(tok >> p.log2_page) - pg_lo];  // all page lookups first: one LDS round trip
    }
#pragma unroll
    for (int q = 0; q < C::KPW; ++q) {
      const int I = min(wave * C::KPW + q, C::NI - 1);
      const int tok = min(tok0 + q_row[q], kv_hi - 1);
      const bool is_k = I * 64 < C::KCH;
      const uint64_t base = is_k ? k_addr : v_addr;
      const uint64_t pgb = is_k ? k_pg_b : v_pg_b;
      const uint32_t inpage = (uint32_t)(tok & pmask) * (is_k ? k_tok_b : v_tok_b) + (is_k ? k_head_b : v_head_b) +
                              q_chunk[q];
      const unsigned char* src =
          (const unsigned char*)(base + ((uint64_t)(uint32_t)pg[q] * (uint32_t)pgb + inpage));
      dma16(src, st + I * 1024);
    }
  };

  // prologue: the first NS-1 tiles in flight
#pragma unroll
  for (int t = 0; t < C::NS - 1; ++t)
    if (t < n_tiles) issue(t, t);

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int stage = tile % C::NS;
    // this wave's loads of `tile` are done once at most (tiles issued after it) * KPW remain
    const int after = min(C::NS - 2, n_tiles - 1 - tile);
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
    ring_barrier();  // every wave's part of `tile` landed; every wave left tile-1's stage
    if (tile + C::NS - 1 < n_tiles) issue(tile + C::NS - 1, (tile + C::NS - 1) % C::NS);

    const unsigned char* kst = smem + stage * C::STAGE;
    const unsigned char* vst = C::VSHARE ? kst : kst + C::KTILE;
    const int tok_w = kv_lo + tile * C::T + wt * C::TT;
    // Per-lane LDS operand addresses are the same every tile; recomputing them
    // (1-2 instructions each) beats keeping ~100 hoisted copies live across the
    // loop, so the lane index is made opaque to loop-invariant code motion here.
    int l16 = l16_in, G4 = G4_in;
    if constexpr (C::LEAN) {
      asm volatile("" : "+v"(l16), "+v"(G4));
      // re-state the ranges the barrier hid (one AND each): with them the
      // swizzle-group mask of every chunk index folds to a constant
      if constexpr (C::FP8) {
        G4 &= 3;
      } else {
        l16 &= 15;
        G4 &= 3;
      }
    }

    // ---- S^T = K Q^T, K rows permuted inside every 32-key chunk
    f32x4 acc[C::RT][C::NNB];
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
      for (int nb = 0; nb < C::NNB; ++nb) acc[rt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      // long head dims: keep the scheduler from hoisting every operand load (register pressure)
      if constexpr (C::NKS > 8) {
        if (ks % 4 == 0) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int nb = 0; nb < C::NNB; ++nb) {
        const int r = wt * C::TT + (nb >> 1) * 32 + 8 * (l16 >> 2) + 4 * (nb & 1) + (l16 & 3);
        bf16x8 a;
        if constexpr (C::FP8) {
          const int cb = 32 * ks + 8 * G4;  // byte offset of the 8 channels inside the row
          const int ch = cb >> 4;
          const u32x2 w = *(const u32x2*)(kst + r * C::KROWB + phys_chunk<C::NCK>(ch, key_k(r)) * 16 + (cb & 15));
          a = e4m3x8_to_bf16x8(w);
        } else {
          // chunk 4 ks + G4 (a row holds 4 NKS chunks)
          a = *(const bf16x8*)(kst + r * C::KROWB + phys_chunk_split<C::NCK, 4>(4 * ks, G4, key_k(r)) * 16);
        }
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
            const int tok = tok_w + (nb >> 1) * 32 + 8 * G4 + 4 * (nb & 1) + e;
            pr[rt][nb][e] = (tok < row_c[rt]) ? s : -INFINITY;
          }
          mx = fmaxf(mx, pr[rt][nb][e]);
        }
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const bool move = mx > m_run[rt] + kRingLazyMax;  // also true on a row's first visible key
      const float m_new = move ? mx : m_run[rt];
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = move ? fast_exp2(m_run[rt] - m_use) : 1.f;
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
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) O[rt][d] *= alpha;
      }
    }

    // ---- O^T += V^T P^T; lane group G4 covers keys 8*G4 .. 8*G4+7 of each 32-key chunk
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
      const int vbase_row = wt * C::TT + 32 * j + 8 * G4;
      auto vkey = [](int r) { return C::VSHARE ? key_k(r) : key_v(r); };
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        if constexpr (C::NDB > 8) {
          if (db % 4 == 0) __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 a;
        if constexpr (C::FP8) {
          // source lane l16 -> key row vbase_row + l16/2, channels 16*db + 8*(l16&1) .. +8
          const int r = vbase_row + (l16 >> 1);
          const unsigned char* src = vst + r * C::VROWB + phys_chunk<C::NCV>(db, vkey(r)) * 16 + (l16 & 1) * 8;
          const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)src));
          a = e4m3x8_to_bf16x8(w);
        } else {
          // source lane l16 -> key rows vbase_row + l16/4 (+4), channels 16*db + 4*(l16&3) .. +4
          // chunk 2 db + (l16 % 4) / 2 (a row holds at least 2 NDB chunks)
          const int hb = (l16 & 3) >> 1;
          const int half = (l16 & 1) * 8;
          const int r1 = vbase_row + (l16 >> 2);
          const int r2 = r1 + 4;
          const unsigned char* p1 = vst + r1 * C::VROWB + phys_chunk_split<C::NCV, 2>(2 * db, hb, vkey(r1)) * 16 + half;
          // vbase_row is a multiple of 8, so r1 has bit 2 clear and key_k(r2) == key_k(r1):
          // with shared rows the second read is the first one 4 rows down
          const unsigned char* p2 =
              C::VSHARE ? p1 + 4 * C::VROWB
                        : vst + r2 * C::VROWB + phys_chunk_split<C::NCV, 2>(2 * db, hb, vkey(r2)) * 16 + half;
          const s16x4 lo = lds_read_tr16(p1);
          const s16x4 hi = lds_read_tr16(p2);
          typedef short s16x8 __attribute__((ext_vector_type(8)));
          const s16x8 a8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          a = __builtin_bit_cast(bf16x8, a8);
        }
#pragma unroll
        for (int rt = 0; rt < C::RT; ++rt) O[rt][db] = mfma16x16x32(a, pb[rt], O[rt][db]);
      }
    }
  }

  // ---- full row sums
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt) {
    l_run[rt] = xor_sum(l_run[rt], 16);
    l_run[rt] = xor_sum(l_run[rt], 32);
  }

  int db_first = 0;
  if constexpr (C::NWT > 1) {
    float* red_ml = (float*)smem;
    f32x4* red_o = (f32x4*)(smem + C::RED_ML);
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
  }

  // ---- epilogue
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
      if (p.counters != nullptr) {
        // read back inside this kernel by a workgroup that may run on another
        // XCD: device-coherent stores that do not stay in this XCD's L2
        if (G4_in == 0 && db_first == 0) st_coherent(p.ws_lse + prow, lse);
        if (!empty) {
          float* dst = p.ws_o + prow * C::DV + G4_in * 4;
#pragma unroll
          for (int d = 0; d < C::NDB; ++d) {
            if (C::NWT > 1 && d % C::NWT != db_first) continue;
            const f32x4 v = O[rt][d] * inv;
#pragma unroll
            for (int j = 0; j < 4; ++j) st_coherent(dst + d * 16 + j, v[j]);
          }
        }
      } else {
      if (G4_in == 0 && db_first == 0) p.ws_lse[prow] = lse;
      if (!empty) {
        float* dst = p.ws_o + prow * C::DV + G4_in * 4;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
          if (C::NWT > 1 && d % C::NWT != db_first) continue;
          *(f32x4*)(dst + d * 16) = O[rt][d] * inv;
        }
      }
      }
    } else {
      if (p.lse_out && G4_in == 0 && db_first == 0) p.lse_out[row_g] = lse;
      if (p.o_dtype == PKV_DTYPE_BF16) {
        __bf16* dst = (__bf16*)p.out + row_t[rt] * p.o_st + row_h[rt] * p.o_sh + G4_in * 4;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
          if (C::NWT > 1 && d % C::NWT != db_first) continue;
          const f32x4 v = O[rt][d] * inv;
          u32x2 w{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2*)(dst + d * 16) = w;
        }
      } else {
        float* dst = (float*)p.out + row_t[rt] * p.o_st + row_h[rt] * p.o_sh + G4_in * 4;
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) {
          if (C::NWT > 1 && d % C::NWT != db_first) continue;
          *(f32x4*)(dst + d * 16) = O[rt][d] * inv;
        }
      }
    }
  }
}

// Workgroup i runs on XCD i % 8, each XCD with its own L2.  With several row
// blocks per (request, KV head), which read the same pages, the grid is laid
// out so that consecutive logical items fall on one XCD and are dispatched one
// after the other: the row blocks of a request then read its pages once from
// memory and again from that XCD's L2, not twice from memory (measured on the
// MLA decode with two speculative rows: 4.98 GB fetched per call before, 2.57
// GB after, for 2.42 GB of KV).
template <class C, bool VT>
__global__ __launch_bounds__(C::NTHR) void attn_dma_kernel(const KParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pages = (int32_t*)(smem + C::LDS);
  const int nx = gridDim.x, ny = gridDim.y;
  const int64_t N = (int64_t)nx * ny * gridDim.z;
  const int64_t P = blockIdx.x + (int64_t)nx * (blockIdx.y + (int64_t)ny * blockIdx.z);
  const int64_t Lg = (p.row_blocks > 1 && N % 8 == 0) ? (P % 8) * (N / 8) + P / 8 : P;
  const int split = (int)(Lg % nx);
  const int y = (int)((Lg / nx) % ny);
  const int z = (int)(Lg / ((int64_t)nx * ny));
  const int span = p.pages_per_split * p.page_size;
  dma_block<C, VT>(p, smem, s_pages, z, y / p.row_blocks, y % p.row_blocks, split * span, split * span + span,
                   split, split == 0);
}

// Fused reducer of the balanced schedule.  Unit u = (request b, KV head g) owns
// the global pages [p_s, p_s + npg); its partial rows come from every workgroup
// whose page range meets that interval, one segment each, in slots w + u.  Each
// such workgroup publishes its partial rows (agent-scope release: the partials
// may sit in another XCD's L2), then increments the unit's counter; the one
// that brings it to the number of owners merges the unit's rows exactly as the
// separate reducer does (L* = max lse_s, w_s = exp(lse_s - L*), out = sum w_s O_s
// / sum w_s) and puts the counter back to zero, so the counter buffer is zero
// between calls (the PR #4557 page: split counters in caller-owned memory that
// reset themselves).  Nothing waits on another workgroup, so there is no
// residency requirement and no spin.
struct StreamUnit {
  int b, g, u;
  int64_t p_s, npg, TP, W;
  // owner workgroup of virtual page q (the w with w*TP/W <= q < (w+1)*TP/W; TP = virtual total)
  __device__ int64_t owner(int64_t q) const { return ((q + 1) * W - 1) / TP; }
  // number of workgroups that own pages of the unit: all of [owner(p_s), owner(p_e)]
  // when every workgroup owns a page (TP >= W), else one per page
  __device__ int count() const { return TP >= W ? (int)(owner(p_s + npg - 1) - owner(p_s) + 1) : (int)npg; }
  __device__ int64_t slot_wg(int k) const { return TP >= W ? owner(p_s) + k : owner(p_s + k); }
};

// The reducer for one unit: every thread owns J items (packed row, 4 value
// channels) and walks the owners in batches of KB with the running-max update
// of the online softmax (m, l, acc rescaled when the max grows), so each batch
// issues all of its loads before the first result is needed.
template <class C, int J, int KB>
__device__ __forceinline__ void merge_unit(const KParams& p, const int* s_slot, const int n, const StreamUnit& su) {
  const int SR = p.slot_rows, G = p.group;
  constexpr int DV4 = C::DV / 4;
  const int nitem = SR * DV4;
  int R[J], c4[J];
  float m[J], l[J];
  f32x4 acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int idx = threadIdx.x + j * C::NTHR;
    R[j] = idx < nitem ? idx / DV4 : 0;
    c4[j] = idx % DV4;
    m[j] = -INFINITY;
    l[j] = 0.f;
    acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int k0 = 0; k0 < n; k0 += KB) {
    float ls[J][KB];
    f32x4 v[J][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int slot = s_slot[min(k0 + kb, n - 1)];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int64_t prow = (int64_t)slot * SR + R[j];
        ls[j][kb] = ld_coherent(p.ws_lse + prow);
        const float* src = p.ws_o + prow * C::DV + 4 * c4[j];
        v[j][kb] = f32x4{ld_coherent(src), ld_coherent(src + 1), ld_coherent(src + 2), ld_coherent(src + 3)};
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int j = 0; j < J; ++j) {
        // owners past n and rows a segment left empty (lse = -inf, O unwritten) do not enter
        const bool live = (k0 + kb < n) && ls[j][kb] != -INFINITY;
        const float mn = live ? fmaxf(m[j], ls[j][kb]) : m[j];
        const float a = (m[j] == -INFINITY) ? 0.f : __expf(m[j] - mn);
        const float w = __expf(ls[j][kb] - mn);
        l[j] = live ? l[j] * a + w : l[j];
        acc[j] = live ? acc[j] * a + w * v[j][kb] : acc[j];
        m[j] = mn;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (threadIdx.x + j * C::NTHR >= nitem) continue;
    const int64_t t = (int64_t)su.b * p.q_len + R[j] / G;
    const int h = su.g * G + R[j] % G;
    float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
    float lse_row = (m[j] == -INFINITY) ? -INFINITY : m[j] + __logf(l[j]);
    if (p.sinks) inv *= fold_sink(lse_row, p.sinks[h]);
    const f32x4 o = acc[j] * inv;
    if (p.o_dtype == PKV_DTYPE_BF16) {
      __bf16* dst = (__bf16*)p.out + t * p.o_st + h * p.o_sh + 4 * c4[j];
      *(u32x2*)dst = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
      *(f32x4*)((float*)p.out + t * p.o_st + h * p.o_sh + 4 * c4[j]) = o;
    }
    if (c4[j] == 0 && p.lse_out) p.lse_out[t * p.num_qo_heads + h] = lse_row;
  }
}

template <class C>
__device__ __forceinline__ void stream_arrive(const KParams& p, unsigned char* smem, int* s_flag,
                                              const StreamUnit& su) {
  // Arrival: every thread releases its partial-row stores at agent scope,
  // the workgroup barrier orders them before thread 0's counter increment
  // (acquire-release at agent scope), and the last arriver's threads acquire
  // at agent scope before reading the other owners' rows.  The rows are
  // written and read with device-coherent accesses as well.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  const int n = su.count();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(p.counters + su.u, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (old + 1 == n);
  }
  __syncthreads();
  if (!*s_flag) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // owner slots into LDS (the ring is idle here; the planner keeps n words within it)
  int* s_slot = (int*)smem;
  for (int k = threadIdx.x; k < n; k += C::NTHR) s_slot[k] = (int)(su.slot_wg(k) + su.u);
  __syncthreads();
  constexpr int DV4 = C::DV / 4;
  const int J = (p.slot_rows * DV4 + C::NTHR - 1) / C::NTHR;  // items (row, 4 channels) per thread
  if (J <= 1) merge_unit<C, 1, 16>(p, s_slot, n, su);
  else if (J <= 2) merge_unit<C, 2, 8>(p, s_slot, n, su);
  else merge_unit<C, 4, 4>(p, s_slot, n, su);
  if (threadIdx.x == 0) __hip_atomic_store(p.counters + su.u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Balanced schedule (see attn_mfma_stream_kernel): equal global page ranges per workgroup.
template <class C, bool VT>
__global__ __launch_bounds__(C::NTHR) void attn_dma_stream_kernel(const KParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pages = (int32_t*)(smem + C::LDS);
  // [B + 1] page prefix, then the reducer's flag word, after the page list(s)
  int32_t* s_pfx = s_pages + p.page_list_cap * (VT ? 2 : 1);
  int* s_flag = s_pfx + p.batch + 1;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int B = p.batch;
  const int cap = p.max_pages_per_seq * p.page_size;
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
  const bool fused = p.counters != nullptr;
  if (!fused && w == 0)
    for (int i = tid; i <= B; i += C::NTHR) p.ws_pfx[i] = s_pfx[i];
  if (fused) {
    // requests with no page are streamed by nobody: their rows are written here
    for (int64_t bb = w; bb < B; bb += W) {
      if (s_pfx[bb + 1] != s_pfx[bb]) continue;
      if (tid == 0) {
        const int L0 = p.seq_lens[bb];
        if (L0 > cap) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_TABLE);
        if (L0 > p.max_kv_len) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_MAXLEN);
        if (L0 < p.q_len) flag_error(p.err_word, PKV_DEVERR_SEQ_LT_QLEN);
      }
      const int nrow = p.q_len * p.num_qo_heads;
      for (int idx = tid; idx < nrow * C::DV; idx += C::NTHR) {
        const int rr = idx / C::DV, d = idx % C::DV;
        const int64_t t = bb * p.q_len + rr / p.num_qo_heads;
        const int h = rr % p.num_qo_heads;
        if (p.o_dtype == PKV_DTYPE_BF16) ((__bf16*)p.out)[t * p.o_st + h * p.o_sh + d] = (__bf16)0.f;
        else ((float*)p.out)[t * p.o_st + h * p.o_sh + d] = 0.f;
        if (d == 0 && p.lse_out) p.lse_out[t * p.num_qo_heads + h] = p.sinks ? p.sinks[h] : -INFINITY;
      }
    }
  }
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
      const bool whole = fused && a == 0 && e == npg;  // sole owner: final rows straight from the epilogue
      dma_block<C, VT>(p, smem, s_pages, b, g, 0, a * p.page_size, e * p.page_size, (int)(w + b * Hkv + g), a == 0,
                   whole);
      if (fused && !whole) {
        StreamUnit su;
        su.b = b;
        su.g = g;
        su.u = b * Hkv + g;
        su.p_s = rs;
        su.npg = npg;
        su.TP = sg.TV;
        su.W = W;
        stream_arrive<C>(p, smem, s_flag, su);
      }
    }
    pos = rs + npg;
  }
}

// ---------------------------------------------------------------- instances
//                           DQK  DV   FP8    VSH    RT NWR NWT TT  NS
using DGqaFp8N2 = DmaCfg<128, 128, true, false, 1, 1, 2, 32, 2>;
using DWideBf16 = DmaCfg<128, 128, false, false, 2, 4, 1, 64, 4>;
using DWideFp8 = DmaCfg<128, 128, true, false, 2, 4, 1, 64, 4>;
// MLA: two 72 KiB stages of 64 keys (one workgroup barrier per 64 keys) fit 252
// VGPRs once the operand addresses are cheap; they beat four 32-key stages
using DMlaBf16 = DmaCfg<576, 512, false, true, 1, 8, 1, 64, 2>;
using DMlaFp8 = DmaCfg<576, 512, true, true, 1, 8, 1, 64, 4>;

template <class C>
static void fill_dma_shape(MfmaShape* s, int waves_per_cu = 8) {
  s->waves_per_cu = waves_per_cu;
  s->rows_per_block = C::ROWS;
  s->tile_tokens = C::T;
  s->threads = C::NTHR;
  s->lds_static = C::LDS;
}

bool dma_shape(int32_t kernel, MfmaShape* s) {
  switch (kernel) {
    // 128-thread groups whose LDS, not registers, limits residency (four per CU)
    case KERNEL_DMA_GQA_FP8_N2: fill_dma_shape<DGqaFp8N2>(s, 16); return true;
    case KERNEL_DMA_WIDE_BF16: fill_dma_shape<DWideBf16>(s); return true;
    case KERNEL_DMA_WIDE_FP8: fill_dma_shape<DWideFp8>(s); return true;
    case KERNEL_DMA_MLA_BF16: fill_dma_shape<DMlaBf16>(s); return true;
    case KERNEL_DMA_MLA_FP8: fill_dma_shape<DMlaFp8>(s); return true;
    default: return false;
  }
}

template <class C, bool VT>
static hipError_t launch_dma_form(const KParams& p, hipStream_t s) {
  static bool attr_done = false;  // idempotent; a race only repeats the same calls
  const size_t extra = (size_t)p.page_list_cap * (VT ? 2 : 1) + (p.stream ? (size_t)p.batch + 2 : 0);
  const size_t lds = C::LDS + ((extra + 3) & ~size_t(3)) * sizeof(int32_t);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_dma_kernel<C, VT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)attn_dma_stream_kernel<C, VT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            160 * 1024);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  if (p.stream) {
    hipLaunchKernelGGL((attn_dma_stream_kernel<C, VT>), dim3(p.num_wg), dim3(C::NTHR), lds, s, p);
  } else {
    dim3 grid(p.num_splits, p.num_kv_heads * p.row_blocks, p.batch);
    hipLaunchKernelGGL((attn_dma_kernel<C, VT>), grid, dim3(C::NTHR), lds, s, p);
  }
  return hipGetLastError();
}

template <class C>
static hipError_t launch_dma_cfg(const KParams& p, hipStream_t s) {
  if (!p.v_table) return launch_dma_form<C, false>(p, s);
  if constexpr (C::VSHARE) {
    return hipErrorInvalidValue;  // V rows are the K rows: the planner never sends a V table here
  } else {
    return launch_dma_form<C, true>(p, s);
  }
}

hipError_t launch_dma(int32_t kernel, const KParams& p, hipStream_t s) {
  switch (kernel) {
    case KERNEL_DMA_GQA_FP8_N2: return launch_dma_cfg<DGqaFp8N2>(p, s);
    case KERNEL_DMA_WIDE_BF16: return launch_dma_cfg<DWideBf16>(p, s);
    case KERNEL_DMA_WIDE_FP8: return launch_dma_cfg<DWideFp8>(p, s);
    case KERNEL_DMA_MLA_BF16: return launch_dma_cfg<DMlaBf16>(p, s);
    case KERNEL_DMA_MLA_FP8: return launch_dma_cfg<DMlaFp8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv

// pkv_attn_mla.hip -- MLA latent decode on v_mfma_f32_32x32x16_bf16, 32 query
// heads per wave, one wave per SIMD.
//
// The PR #4557 page's MLA decode: every query head (times the speculative
// rows) reads one latent KV head whose 576-channel rows hold 512 latent and 64
// rope channels, and V is the latent part of the same row, so one K tile in
// LDS serves both products.  The work per key and head is 576 + 512 MACs
// against 1152 bytes of KV per key shared by all heads: decode with one query
// row is HBM-bound only if the matrix cores keep up at about half their peak
// at the same time, so the tiling is chosen for the matrix cores and LDS:
//   * a wave owns 32 packed query rows (heads) and the whole 512-wide output
//     of those rows (256 accumulator registers), with its 36 Q operand
//     registers resident: every K operand read from LDS feeds one 32x32x16
//     MFMA (1 KiB of LDS per 32 Ki MACs), every V^T operand one more;
//     measured on gfx950 the LDS serves ds_read_b128 at 256 bytes per clock
//     per CU, twice what four such waves at full matrix rate read;
//   * S^T = K Q^T and O^T += V^T P^T with the query rows on the column axis;
//     A rows of S^T read keys with index bits 2 and 3 exchanged, which makes
//     result elements 8s..8s+7 of a lane the B operand of the s-th 16-key step
//     of the PV product (P^T never crosses lanes);
//   * keys arrive in 32-key blocks (36 KiB, one per ring stage, four stages)
//     through global_load_lds_dwordx4 into LDS; row r's 16-byte chunk c is
//     stored at c ^ key(r): the latent chunks use a 4-bit key that spreads the
//     sixteen rows one ds_read_b128 serves, and the four rows of each half of a
//     transposed V read, over all 64 banks (odd rows of 1152 bytes start half
//     a bank row later), the rope chunks a 3-bit key;
//   * one MFMA sequence per block carries two independent products, the S^T
//     product of block j+1 (first) and the PV product of block j, and the
//     softmax of block j+1 runs in pieces between the PV steps that follow
//     its last S^T step; the running maximum moves only on jumps of more
//     than 8 (log2 units), so O is rescaled rarely.
// Paging follows the flashinfer.cake_fmha API page's contract (key j of
// request b is token j % P of page block_tables[b][j / P]); Split-KV partials
// (normalized O and natural-log LSE) go to the caller's workspace for the
// separate reducer as the PR #4557 page describes.

#include <cfloat>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"
#include "pkv_ring.h"

namespace pkv {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace mla {

constexpr int DQK = 576, DV = 512;
constexpr int ROWB = DQK * 2;     // bytes of one 576-channel row in the pool
constexpr int LATB = DV * 2;      // LDS: the latent part of a row (64 chunks) ...
constexpr int ROPEB = ROWB - LATB;  // ... and its rope part (8 chunks) in a region of their own
constexpr int NKS = DQK / 16;     // 36 k-steps of S^T
constexpr int NDB = DV / 32;      // 16 value blocks of O^T
constexpr int NW = 4;             // waves per workgroup (one per SIMD)
constexpr int NTHR = 64 * NW;
constexpr int ROWS = 32 * NW;     // packed query rows per workgroup
constexpr int BK = 32;            // keys per block and per ring stage
constexpr int STAGE = BK * ROWB;  // 36 KiB: 32 latent rows of 1 KiB, then 32 rope rows of 128 bytes
constexpr int ROPE_OFF = BK * LATB;
constexpr int NI = BK + BK * ROPEB / 1024;  // 36 wave-instructions fill a stage: one per latent row, 4 for the rope
constexpr int KPW = NI / NW;      // 9 per wave
constexpr int NS = 4;             // ring stages
constexpr int LDS = NS * STAGE;   // 144 KiB
// Read-ahead of the operand rings: 3 measured about 1 % faster than 4 at one
// query row (B512 L4096 q=1, four alternating pairs on one box; two query rows
// unchanged), and 5 or 6 no faster than 4 (the chip is at its power limit)
#ifndef PKV_MLA_PD
#define PKV_MLA_PD 3
#endif
#ifndef PKV_MLA_PDV
#define PKV_MLA_PDV PKV_MLA_PD
#endif
constexpr int PDK = PKV_MLA_PD;   // K operand reads issued this many MFMAs ahead
constexpr int PDV = PKV_MLA_PDV;  // V^T operand reads issued this many MFMAs ahead
constexpr float kLazy = 8.f;  // largest rise of a row max (log2 units) absorbed without rescaling O
static_assert(NI % NW == 0 && KPW * (NS - 1) < 64 && LATB == 1024 && BK * ROPEB == NW * 1024, "ring geometry");

// Chunk keys (16-byte chunk c of row r is stored at c ^ key(r); XOR is its own
// inverse).  Latent rows are 1 KiB apart, so only the key separates the
// banks: the sixteen rows one ds_read_b128 serves get sixteen keys, and the
// four consecutive rows of each half of a transposed V read keys that differ
// in bits 2-3 (their four chunks then fill 256 distinct bytes).  Rope rows are
// 128 bytes apart: odd rows sit half a bank row later, and the 3-bit key
// spreads each parity class over the other eight slots.
__device__ __forceinline__ int key_lat(int r) { return 4 * (r & 3) | ((r >> 2) & 3); }
__device__ __forceinline__ int key_rope(int r) { return (r >> 1) & 7; }
// key read by A row r of S^T: bits 2 and 3 exchanged
__device__ __forceinline__ int perm(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The MFMAs are issued through inline assembly so that their register
// classes are fixed: the 256 output accumulators in AGPRs ("a"), the S^T
// accumulator, the operands and everything else in VGPRs ("v").  With one
// wave per SIMD the compiler gives every MFMA the AGPR form, and the S^T
// accumulator then cannot live beside the outputs.  The compiler does not
// look inside an asm statement, so the wait states the hardware needs around
// these MFMAs are written out here: two before a product whose B operand a
// vector instruction has just written, sixteen between the last S^T step and
// the vector instructions that read its result, sixteen before vector
// instructions read or rewrite the AGPR outputs and four after they did.
// Steps accumulating into the same registers back to back need none.
__device__ __forceinline__ void mfma_s_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s_last(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7" : "+v"(acc) : "v"(a), "v"(b));
}
template <bool B_FRESH>
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& a, const bf16x8& b) {
  if constexpr (B_FRESH)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}
// wait states around vector access to the AGPR outputs (the asm operands tie
// every accumulator to the fence, so no access moves across it)
template <int NOPS>
__device__ __forceinline__ void o_fence(f32x16 (&O)[NDB]) {
  static_assert(NDB == 16, "sixteen value blocks");
  if constexpr (NOPS >= 16)
    asm volatile("s_nop 7\n\ts_nop 7"
                 : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]), "+a"(O[6]), "+a"(O[7]),
                   "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]), "+a"(O[12]), "+a"(O[13]), "+a"(O[14]),
                   "+a"(O[15]));
  else
    asm volatile("s_nop 3"
                 : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]), "+a"(O[6]), "+a"(O[7]),
                   "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]), "+a"(O[12]), "+a"(O[13]), "+a"(O[14]),
                   "+a"(O[15]));
}

// Slot of S^T step ks in the two-stream MFMA sequence of a block (68 slots:
// 36 S^T steps, 32 PV steps): seven S^T steps, then one PV step, so the S^T
// product ends at slot 40 and the softmax runs beside the remaining PV steps.
constexpr int s_slot(int ks) { return ks + ks / 7; }
constexpr int s_step_at(int t) {
  for (int ks = 0; ks < NKS; ++ks)
    if (s_slot(ks) == t) return ks;
  return -1;
}
constexpr int s_steps_before(int t) {
  int n = 0;
  for (int ks = 0; ks < NKS; ++ks) n += s_slot(ks) < t;
  return n;
}
static_assert(s_slot(NKS - 1) == 40 && s_steps_before(68) == NKS, "slot map");

// orders vector access to one block of AGPR outputs (no instructions)
__device__ __forceinline__ void o_touch(f32x16& o) { asm volatile("" : "+a"(o)); }

}  // namespace mla

__global__ __launch_bounds__(mla::NTHR, 1) void attn_mla32_kernel(const KParams p) {
  using namespace mla;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  int32_t* s_pages = (int32_t*)(smem + LDS);

  // Workgroup i runs on XCD i % 8: the row blocks of one request (speculative
  // rows) are placed on one XCD back to back so the later ones read its pages
  // from that XCD's L2.
  const int nx = gridDim.x, ny = gridDim.y;
  const int64_t N = (int64_t)nx * ny * gridDim.z;
  const int64_t Pl = blockIdx.x + (int64_t)nx * (blockIdx.y + (int64_t)ny * blockIdx.z);
  const int64_t Lg = (p.row_blocks > 1 && N % 8 == 0) ? (Pl % 8) * (N / 8) + Pl / 8 : Pl;
  const int split = (int)(Lg % nx);
  const int y = (int)((Lg / nx) % ny);
  const int b = (int)(Lg / ((int64_t)nx * ny));
  const int g = y / p.row_blocks, rblk = y % p.row_blocks;
  const int span_s = p.pages_per_split * p.page_size;
  const int part_lo = split * span_s, part_hi = part_lo + span_s;
  const bool lead = split == 0;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tid = threadIdx.x;
  const int h = lane >> 5;    // k half of the operands
  const int c32 = lane & 31;  // query row of the wave
  const int G = p.group;

  int t0, n_b;
  if (p.is_context) {
    const int a0 = p.q_indptr[b], a1 = p.q_indptr[b + 1];
    if (a0 < 0 || a1 < a0 || a1 - a0 > p.max_q_len || a1 > p.total_q) {
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
  const int row0 = rblk * ROWS;
  if (row0 >= row_space) return;

  int L = p.seq_lens[b];
  if (lead && g == 0 && rblk == 0 && tid == 0) {
    if (L > p.max_pages_per_seq * p.page_size) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_TABLE);
    if (L > p.max_kv_len) flag_error(p.err_word, PKV_DEVERR_SEQ_GT_MAXLEN);
    if (L < n_b) flag_error(p.err_word, PKV_DEVERR_SEQ_LT_QLEN);
  }
  L = max(0, min(L, p.kv_span));

  const int last_row = min(row0 + ROWS, row_space) - 1;
  const int c_max = p.causal ? min(L, max(0, L - n_b + last_row / G + 1)) : L;
  const int kv_lo = part_lo;
  const int kv_hi = min(part_hi, c_max);
  const int nblk = kv_hi > kv_lo ? (kv_hi - kv_lo + BK - 1) / BK : 0;
  const bool split_mode = p.ws_o != nullptr;
  if (nblk == 0 && split_mode) return;  // a partition the reducer never reads

  // the partition's validated page list: LDS, then registers (lane l of pl[k]
  // holds page 64k + l; the planner keeps a partition within 64 kPageRegs pages)
  constexpr int kPageRegs = kM32MaxPages / 64;
  const int pg_lo = kv_lo >> p.log2_page;
  const int n_pg = nblk > 0 ? ((kv_hi - 1) >> p.log2_page) - pg_lo + 1 : 0;
  for (int i = tid; i < n_pg; i += NTHR) {
    int pg = p.table[(int64_t)b * p.table_stride + pg_lo + i];
    if (p.num_pages > 0 && (pg < 0 || pg >= p.num_pages)) {
      flag_error(p.err_word, PKV_DEVERR_PAGE_RANGE);
      pg = min(max(pg, 0), p.num_pages - 1);
    }
    s_pages[i] = pg;
  }

  const float k_scale = p.k_scale_dev ? *p.k_scale_dev : p.k_scale;
  const float v_scale = p.v_scale_dev ? *p.v_scale_dev : p.v_scale;
  const float sc2_raw = p.scale * k_scale * kLog2e;
  // a negative logit scale is folded into Q (an exact bf16 sign flip), so the
  // softmax only ever needs the row max of the raw products
  const float sc2 = fmaxf(fabsf(sc2_raw), FLT_MIN);  // > 0: a masked key's -inf score stays -inf
  const uint32_t q_sign = sc2_raw < 0.f ? 0x80008000u : 0u;

  // ---- this lane's query row and its Q operands (B of S^T: row c32, channels 16 ks + 8 h .. +7)
  const int R = row0 + wave * 32 + c32;
  const bool row_ok = R < row_space;
  const int qi = row_ok ? R / G : 0;
  const int row_t = t0 + qi;
  const int row_h = g * G + (row_ok ? R % G : 0);
  const int row_c = row_ok ? min(max(p.causal ? L - n_b + qi + 1 : L, 0), kv_hi) : 0;
  bf16x8 qB[NKS];
  {
    // rows past the request read a valid row (their results are never stored)
    const __bf16* qrow = (const __bf16*)p.q + row_t * p.q_st + row_h * p.q_sh + 8 * h;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 q = *(const bf16x8*)(qrow + 16 * ks);
      u32x4 qw = __builtin_bit_cast(u32x4, q);
      qw ^= u32x4{q_sign, q_sign, q_sign, q_sign};
      qB[ks] = __builtin_bit_cast(bf16x8, qw);
    }
  }
  // blocks ending at or below c_lo need no mask for any row of the wave; blocks
  // at or past c_hi hold no key any of its rows sees
  const int c_lo = __builtin_amdgcn_readfirstlane(-wave_max_i(row_ok ? -row_c : INT_MIN + 1));
  const int c_hi = __builtin_amdgcn_readfirstlane(wave_max_i(row_c));

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 O[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d)
#pragma unroll
    for (int e = 0; e < 16; ++e) O[d][e] = 0.f;

  __syncthreads();  // page list visible
  int pl[kPageRegs];
#pragma unroll
  for (int k = 0; k < kPageRegs; ++k) pl[k] = 64 * k + lane < n_pg ? s_pages[64 * k + lane] : 0;
  auto page_of = [&](int idx) -> uint32_t {
    int v = __builtin_amdgcn_readlane(pl[0], idx & 63);
#pragma unroll
    for (int k = 1; k < kPageRegs; ++k)
      if ((idx >> 6) == k) v = __builtin_amdgcn_readlane(pl[k], idx & 63);
    return (uint32_t)v;
  };

  // ---- loader: wave-instruction I of a stage fills its 16-byte slots 64 I ..
  // 64 I + 63 (row r = slot / 72, physical chunk slot % 72); lane l fetches the
  // logical chunk stored in slot 64 I + l.  A block lies inside one page (the
  // planner requires page sizes that are multiples of 32), so the page base is
  // wave-uniform (SADDR form) and a lane supplies its 32-bit in-page offset.
  // Rows past the visible keys reload the last visible key (a finite row that
  // the softmax then weighs zero), so page tails never reach LDS.
  const uint32_t k_tok_b = (uint32_t)(p.k_stok * 2);
  const uint64_t k_base = (uint64_t)p.k + (uint64_t)g * (uint64_t)p.k_sh * 2;
  const uint64_t k_pg_b = (uint64_t)p.k_sp * 2;
  const int pmask = p.page_size - 1;
  // A block's KPW instructions per wave go out as one burst right after the
  // barrier that frees their stage.  Measured on gfx950 (shader-clock stamps
  // per block): the burst stalls the issuing wave about 63 ticks per
  // instruction, the rate at which the CU accepts them from four waves at
  // once; the same instructions placed one at a time between the MFMAs of the
  // next S^T product cost about 160 ticks each.
  // Instruction q < KPW - 1 of wave w fills latent row r = (KPW - 1) w + q
  // (lane l fetches logical chunk l ^ key_lat(r), so the row's offset is
  // uniform and a lane adds one XOR); instruction KPW - 1 fills the rope
  // rows 8 w .. 8 w + 7 (lane l: row 8 w + l / 8, chunk 64 + (l % 8) ^ key).
  auto issue = [&](int blk, int stage) {
    const int tok0 = kv_lo + blk * BK;
    const uint64_t sbase = k_base + (uint64_t)page_of((tok0 >> p.log2_page) - pg_lo) * k_pg_b;
    unsigned char* st = smem + stage * STAGE;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed per block rather than kept live
    ln &= 63;
#pragma unroll
    for (int q = 0; q < KPW; ++q) {
      if (q < KPW - 1) {
        const int r = wave * (KPW - 1) + q;  // wave-uniform
        const int tok = min(tok0 + r, kv_hi - 1);
        const uint64_t rbase = sbase + (uint64_t)((uint32_t)(tok & pmask) * k_tok_b);
        dma16_saddr(rbase, (uint32_t)((ln ^ key_lat(r)) * 16), st + r * LATB);
      } else {
        const int r = 8 * wave + (ln >> 3);
        const int tok = min(tok0 + r, kv_hi - 1);
        const uint32_t voff = (uint32_t)(tok & pmask) * k_tok_b + (uint32_t)(LATB + 16 * ((ln & 7) ^ key_rope(r)));
        dma16_saddr(sbase, voff, st + ROPE_OFF + wave * 1024);
      }
    }
  };

  // ---- per-lane operand geometry.  The offsets are recomputed at every
  // product from a lane index the compiler cannot see through: kept live
  // across the loop they would be one register per read (about a hundred).
  auto opaque_lane = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln & 63;
  };
  auto stage_of = [&](int j) { return smem + (j % NS) * STAGE; };
  // K operand of k-step ks for A row ln % 32 of S^T: key perm(ln % 32),
  // logical chunk 2 ks + ln / 32; the chunk's swizzle only touches the low
  // bits, so a product needs 8 latent and 4 rope lane offsets, the rest is
  // an immediate
  struct KGeo {
    const unsigned char* lat;  // latent row of this lane's key
    const unsigned char* rope;  // its rope row
    int lo[8], ro[4];
  };
  auto k_geo = [&](int j) {
    const int ln = opaque_lane();
    const int kkey = perm(ln & 31), hh = ln >> 5;
    KGeo k;
    k.lat = stage_of(j) + kkey * LATB;
    k.rope = stage_of(j) + ROPE_OFF + kkey * ROPEB;
    const int kl = key_lat(kkey), kr = key_rope(kkey);
#pragma unroll
    for (int t = 0; t < 8; ++t) k.lo[t] = 16 * ((2 * t + hh) ^ kl);
#pragma unroll
    for (int t = 0; t < 4; ++t) k.ro[t] = 16 * ((2 * t + hh) ^ kr);
    return k;
  };
  auto k_read = [&](const KGeo& k, int ks) -> bf16x8 {
    const int c = 2 * ks;  // + hh
    if (c < 64) return *(const bf16x8*)(k.lat + k.lo[(c & 15) >> 1] + 256 * (c >> 4));
    return *(const bf16x8*)(k.rope + k.ro[(c & 7) >> 1]);
  };
  // V^T transpose reads: 16-lane group q = lane / 16 covers values 16 (q & 1) ..
  // +15 and keys 8 (q >> 1) + 4 half + (lane % 16) / 4 of a 16-key step; source
  // lane j = lane % 16 supplies 4 values of one key row at value offset 4 (j % 4).
  // key_lat of the rows vrow + 4 half + 16 st depends on half only through bit 0.
  static_assert(ROWB == 1152, "the V^T geometry below uses latent rows of 1 KiB");
  struct VGeo {
    const unsigned char* row;
    int off[2][4];  // [half][db % 4]
  };
  auto v_geo = [&](int j) {
    const int ln = opaque_lane();
    const int vj = ln & 15, vq = ln >> 4;
    const int vrow = 8 * (vq >> 1) + (vj >> 2);
    const int vc_lane = 2 * (vq & 1) + ((vj & 3) >> 1);
    VGeo v;
    v.row = stage_of(j) + vrow * LATB + 8 * (vj & 1);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int key = key_lat(vrow + 4 * hf);
#pragma unroll
      for (int t = 0; t < 4; ++t) v.off[hf][t] = 4 * hf * LATB + 16 * ((4 * t + vc_lane) ^ key);
    }
    return v;
  };
  auto v_read = [&](const VGeo& v, int i) -> bf16x8 {  // i = 2 db + st
    const int db = i >> 1, st = i & 1;
    const unsigned char* src = v.row + 16 * st * LATB + 256 * (db >> 2);
    const s16x4 lo = lds_read_tr16(src + v.off[0][db & 3]);
    const s16x4 hi = lds_read_tr16(src + v.off[1][db & 3]);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
  };

  // S^T of block j: K operand reads PDK steps ahead of their MFMAs
  auto s_product = [&](int j, f32x16& acc, auto&& step_work) {
    const KGeo blk = k_geo(j);
    bf16x8 ring[PDK];
#pragma unroll
    for (int q = 0; q < PDK; ++q) ring[q] = k_read(blk, q);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8 a = ring[ks % PDK];
      if (ks + PDK < NKS) ring[ks % PDK] = k_read(blk, ks + PDK);
      if (ks == 0) mfma_s_first(acc, a, qB[ks]);
      else if (ks == NKS - 1) mfma_s_last(acc, a, qB[ks]);
      else mfma_s(acc, a, qB[ks]);
      step_work(ks);
    }
  };
  // O^T += V^T P^T of block j, the 16-key steps outermost (an output block is
  // revisited 16 MFMAs later, never back to back).  `step_work(i)` runs after
  // the i-th MFMA: vector work that shares this region.
  auto pv_product = [&](int j, const bf16x8 (&pb)[2], bool pb_fresh, auto&& step_work) {
    const VGeo blk = v_geo(j);
    constexpr int NV = 2 * NDB;
    bf16x8 ring[PDV];
#pragma unroll
    for (int q = 0; q < PDV; ++q) ring[q] = v_read(blk, 2 * (q % NDB) + q / NDB);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int st = i / NDB, db = i % NDB;
      const bf16x8 a = ring[i % PDV];
      if (i + PDV < NV) ring[i % PDV] = v_read(blk, 2 * ((i + PDV) % NDB) + (i + PDV) / NDB);
      if (pb_fresh && (i == 0 || i == NDB)) mfma_o<true>(O[db], a, pb[st]);
      else mfma_o<false>(O[db], a, pb[st]);
      step_work(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no_work = [](int) {};
  // Online softmax of block j (exp2 domain).  Element e of acc holds key
  // 16 (e / 8) + 8 h + e % 8 of the block for this lane's query row; the
  // other 16 keys of the row sit in lane l ^ 32.  Part 1: the row max, the new
  // reference and alpha; part 2: the weights (in place), the lane's share of
  // the row sum and the P^T operand of the PV product.
  auto softmax_max = [&](auto full_tag, int j, f32x16& acc, float& m_use, float& alpha, bool& moved) {
    constexpr bool FULL = decltype(full_tag)::value;
    float mx;
    if constexpr (FULL) {
      float mr = acc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mr = fmaxf(mr, acc[e]);
      mx = half_swap_max(mr) * sc2;
    } else {
      const int blk_tok = kv_lo + j * BK;
      mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int tok = blk_tok + 16 * (e >> 3) + 8 * h + (e & 7);
        acc[e] = tok < row_c ? acc[e] * sc2 : -INFINITY;
        mx = fmaxf(mx, acc[e]);
      }
      mx = half_swap_max(mx);
    }
    moved = mx > m_run + kLazy;  // also true on a row's first visible key
    const float m_new = moved ? mx : m_run;
    m_use = (m_new == -INFINITY) ? 0.f : m_new;
    alpha = moved ? fast_exp2(m_run - m_use) : 1.f;
    m_run = m_new;
  };
  auto weight = [&](auto full_tag, f32x16& acc, int e, float m_use) {
    constexpr bool FULL = decltype(full_tag)::value;
    acc[e] = FULL ? fast_exp2(fmaf(acc[e], sc2, -m_use)) : fast_exp2(acc[e] - m_use);
  };
  auto pack = [&](const f32x16& acc, bf16x8 (&pb)[2]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const u32x4 wv{pack_bf16x2(acc[8 * st + 0], acc[8 * st + 1]), pack_bf16x2(acc[8 * st + 2], acc[8 * st + 3]),
                     pack_bf16x2(acc[8 * st + 4], acc[8 * st + 5]), pack_bf16x2(acc[8 * st + 6], acc[8 * st + 7])};
      pb[st] = __builtin_bit_cast(bf16x8, wv);
    }
  };
  auto softmax_exp = [&](auto full_tag, f32x16& acc, float m_use, float alpha, bf16x8 (&pb)[2]) {
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      weight(full_tag, acc, e, m_use);
      ls += acc[e];
    }
    l_run = fmaf(l_run, alpha, ls);
    pack(acc, pb);
  };
  auto rescale = [&](bool moved, float alpha) {
    if (__builtin_amdgcn_ballot_w64(moved) != 0) {
      o_fence<16>(O);
#pragma unroll
      for (int d = 0; d < NDB; ++d) {  // one block at a time: 16 staging registers, not 256
        o_touch(O[d]);
        O[d] *= alpha;
        o_touch(O[d]);
      }
      o_fence<4>(O);
    }
  };
  auto active = [&](int j) { return kv_lo + j * BK < c_hi; };
  auto full_block = [&](int j) { return kv_lo + j * BK + BK <= c_lo; };
  // this wave's loads of block j are complete once at most (blocks issued
  // after j) * KPW remain
  auto wait_block = [&](int after) {
    if (after >= 2) wait_loads<2 * KPW>();
    else if (after == 1) wait_loads<KPW>();
    else wait_loads<0>();
  };

#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < nblk) issue(t, t);
  f32x16 acc;
  bf16x8 pb_prev[2], pb_cur[2];
  if (nblk > 0) {
    wait_block(min(NS - 2, nblk - 1));
    ring_barrier();
    if (active(0)) s_product(0, acc, no_work);
  }
  // Two streams on the matrix core: step j runs the S^T product of block
  // j+1 and the PV product of block j in one sequence, MFMA by MFMA, so
  // each stream's LDS operand reads get longer to arrive.  The S^T steps
  // come first (ks + ks / 7: seven S^T steps, then one PV step), and the
  // softmax of block j+1 runs in pieces between the PV steps that follow,
  // in the shadow of their MFMAs; the rare O rescale comes after the last.
  // Each piece ties its results to an empty asm statement, which keeps it
  // between the MFMA statements around it (the compiler would otherwise
  // sink the arithmetic to its first use after the sequence).
  float sm_mx = 0.f, sm_use = 0.f, sm_alpha = 1.f, sm_ls = 0.f;
  bool sm_moved = false;
  auto softmax_piece = [&](auto piece, int jS, bool full) {
    constexpr int c = decltype(piece)::value;
    if constexpr (c == 0) {
      if (!full) {  // keys at or past a row's causal limit weigh zero (sc2 > 0)
        const int blk_tok = kv_lo + jS * BK;
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (blk_tok + 16 * (e >> 3) + 8 * h + (e & 7) >= row_c) acc[e] = -INFINITY;
      }
      sm_mx = acc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) sm_mx = fmaxf(sm_mx, acc[e]);
      asm volatile("" : "+v"(sm_mx));
    } else if constexpr (c == 1) {
#pragma unroll
      for (int e = 8; e < 16; ++e) sm_mx = fmaxf(sm_mx, acc[e]);
      asm volatile("" : "+v"(sm_mx));
    } else if constexpr (c == 2) {
      const float mx = half_swap_max(sm_mx) * sc2;
      sm_moved = mx > m_run + kLazy;  // also true on a row's first visible key
      const float m_new = sm_moved ? mx : m_run;
      sm_use = (m_new == -INFINITY) ? 0.f : m_new;
      sm_alpha = sm_moved ? fast_exp2(m_run - sm_use) : 1.f;
      m_run = m_new;
      sm_ls = 0.f;
      asm volatile("" : "+v"(sm_use), "+v"(sm_alpha), "+v"(m_run));
    } else if constexpr (c < 19) {
      constexpr int e = c - 3;
      acc[e] = fast_exp2(fmaf(acc[e], sc2, -sm_use));
      sm_ls += acc[e];
      asm volatile("" : "+v"(acc[e]), "+v"(sm_ls));
    } else {
      l_run = fmaf(l_run, sm_alpha, sm_ls);
      pack(acc, pb_cur);
      asm volatile("" : "+v"(pb_cur[0]), "+v"(pb_cur[1]), "+v"(l_run));
    }
  };
  constexpr int kPieces = 20;
  auto dual_product = [&](int jS, int jP, const bf16x8 (&pb)[2]) {
    const bool full = full_block(jS);
    const KGeo kg = k_geo(jS);
    const VGeo vg = v_geo(jP);
    constexpr int NV = 2 * NDB;
    constexpr int NSLOT = NKS + NV;
    bf16x8 kr[PDK], vr[PDV];
#pragma unroll
    for (int q = 0; q < PDK; ++q) kr[q] = k_read(kg, q);
#pragma unroll
    for (int q = 0; q < PDV; ++q) vr[q] = v_read(vg, 2 * (q % NDB) + q / NDB);
    static_for<0, NSLOT>([&](auto slot) {
      constexpr int t = decltype(slot)::value;
      constexpr int ks_here = s_step_at(t);
      if constexpr (ks_here >= 0) {
        constexpr int ks = ks_here;
        const bf16x8 a = kr[ks % PDK];
        if (ks + PDK < NKS) kr[ks % PDK] = k_read(kg, ks + PDK);
        if (ks == 0) mfma_s_first(acc, a, qB[ks]);
        else if (ks == NKS - 1) mfma_s_last(acc, a, qB[ks]);
        else mfma_s(acc, a, qB[ks]);
      } else {
        constexpr int i = t - s_steps_before(t);
        constexpr int st = i / NDB, db = i % NDB;
        const bf16x8 a = vr[i % PDV];
        if (i + PDV < NV) vr[i % PDV] = v_read(vg, 2 * ((i + PDV) % NDB) + (i + PDV) / NDB);
        if (i == 0 || i == NDB) mfma_o<true>(O[db], a, pb[st]);
        else mfma_o<false>(O[db], a, pb[st]);
        // softmax piece c at slot first + c (NSLOT - 2 - first) / (kPieces - 1):
        // the last piece writes P^T of block j+1 before the last MFMA reads
        // P^T of block j, so the two never share registers
        constexpr int first = s_slot(NKS - 1) + 1;
        constexpr int span = NSLOT - 2 - first;
        static_for<0, kPieces>([&](auto piece) {
          constexpr int c = decltype(piece)::value;
          if constexpr (first + (c * span) / (kPieces - 1) == t) softmax_piece(piece, jS, full);
        });
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto softmax_block = [&](int j) {
    float m_use = 0.f, alpha = 1.f;
    bool moved = false;
    if (full_block(j)) {
      softmax_max(std::true_type{}, j, acc, m_use, alpha, moved);
      softmax_exp(std::true_type{}, acc, m_use, alpha, pb_cur);
    } else {
      softmax_max(std::false_type{}, j, acc, m_use, alpha, moved);
      softmax_exp(std::false_type{}, acc, m_use, alpha, pb_cur);
    }
    rescale(moved, alpha);
  };
  // block 0: its S^T ran above; every later block is computed even where
  // it holds no key a row of this wave sees (the masked softmax then
  // weighs it zero), so the loop has one product call site
  if (nblk > 0) softmax_block(0);
  for (int j = 0; j + 1 < nblk; ++j) {
    pb_prev[0] = pb_cur[0];
    pb_prev[1] = pb_cur[1];
    wait_block(min(1, nblk - 2 - j));
    ring_barrier();  // block j+1 landed; every wave finished reading block j-1's stage
    if (j + NS - 1 < nblk) issue(j + NS - 1, (j + NS - 1) % NS);  // into block j-1's stage
    dual_product(j + 1, j, pb_prev);
    rescale(sm_moved, sm_alpha);
  }
  if (nblk > 0) pv_product(nblk - 1, pb_cur, true, no_work);
  o_fence<16>(O);  // the last MFMAs' outputs before the epilogue reads them

  // ---- epilogue: element e of O[db] is value 32 db + 8 (e / 4) + 4 h + e % 4 of row c32
  l_run = half_swap_sum(l_run);
  if (!row_ok) return;
  const bool empty = !(l_run > 0.f);
  float inv = empty ? 0.f : v_scale / l_run;
  float lse = empty ? -INFINITY : (m_run * kLn2 + __logf(l_run));
  if (p.sinks && !split_mode) inv *= fold_sink(lse, p.sinks[row_h]);  // split: the reducer adds it
  const int64_t row_g = (int64_t)row_t * p.num_qo_heads + row_h;
#pragma unroll
  for (int d = 0; d < NDB; ++d) o_touch(O[d]);  // read out one block at a time below
  if (split_mode) {
    const int64_t prow = (int64_t)split * p.rows_total + row_g;
    if (h == 0) p.ws_lse[prow] = lse;
    if (!empty) {
      float* dst = p.ws_o + prow * DV + 4 * h;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4*)(dst + 32 * d + 8 * q) = f32x4{O[d][4 * q], O[d][4 * q + 1], O[d][4 * q + 2], O[d][4 * q + 3]} * inv;
    }
  } else {
    if (p.lse_out && h == 0) p.lse_out[row_g] = lse;
    if (p.o_dtype == PKV_DTYPE_BF16) {
      __bf16* dst = (__bf16*)p.out + row_t * p.o_st + row_h * p.o_sh + 4 * h;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 wv{pack_bf16x2(O[d][4 * q] * inv, O[d][4 * q + 1] * inv),
                         pack_bf16x2(O[d][4 * q + 2] * inv, O[d][4 * q + 3] * inv)};
          *(u32x2*)(dst + 32 * d + 8 * q) = wv;
        }
    } else {
      float* dst = (float*)p.out + row_t * p.o_st + row_h * p.o_sh + 4 * h;
#pragma unroll
      for (int d = 0; d < NDB; ++d)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f32x4*)(dst + 32 * d + 8 * q) = f32x4{O[d][4 * q], O[d][4 * q + 1], O[d][4 * q + 2], O[d][4 * q + 3]} * inv;
    }
  }
}

bool mla32_shape(int32_t kernel, MfmaShape* s) {
  if (kernel != KERNEL_MLA32_BF16) return false;
  s->rows_per_block = mla::ROWS;
  s->tile_tokens = mla::BK;
  s->threads = mla::NTHR;
  s->lds_static = mla::LDS;
  s->waves_per_cu = 4;
  return true;
}

hipError_t launch_mla32(int32_t kernel, const KParams& p, hipStream_t s) {
  if (kernel != KERNEL_MLA32_BF16) return hipErrorInvalidValue;
  static bool attr_done = false;  // idempotent; a race only repeats the same call
  const size_t lds = mla::LDS + (((size_t)p.page_list_cap + 3) & ~size_t(3)) * sizeof(int32_t);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mla32_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       160 * 1024);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  dim3 grid(p.num_splits, p.num_kv_heads * p.row_blocks, p.batch);
  hipLaunchKernelGGL(attn_mla32_kernel, grid, dim3(mla::NTHR), lds, s, p);
  return hipGetLastError();
}

}  // namespace pkv

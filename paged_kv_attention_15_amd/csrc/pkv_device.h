// pkv_device.h -- device-side building blocks for the gfx950 paged-KV kernels.
//
// Storage decoding (bf16, OCP e4m3), wavefront reductions, the 16x16x32 bf16
// MFMA wrapper and the LDS transpose read.  Operand layouts below were
// measured on gfx950 (see the kernel comments for how each is used):
//   v_mfma_f32_16x16x32_bf16  A: lane l holds row l%16, k = 8*(l/16)+e (e=0..7)
//                             B: lane l holds col l%16, k = 8*(l/16)+e
//                             C: lane l, element e is (row 4*(l/16)+e, col l%16)
//   ds_read_b64_tr_b16        inside each 16-lane group, lane i receives
//                             element i%4 of the 8-byte rows addressed by lanes
//                             (i/4) + 4k, k = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- decoding
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// two e4m3 bytes (selected half of a 32-bit word) -> two bf16 (exact: e4m3 is a subset of bf16)
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16x2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HI);
}

// two e4m3 bytes -> two fp32
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32x2(uint32_t word) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(word, HI);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  f32x2 v = e4m3x2_to_f32x2<false>(byte & 0xFFu);
  return v[0];
}

// 16 e4m3 codes (one 16-byte load) -> 16 bf16 (two 16-byte LDS chunks)
__device__ __forceinline__ void e4m3x16_to_bf16x16(u32x4 src, u32x4& lo, u32x4& hi) {
  bf16x2 t[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    t[2 * w] = e4m3x2_to_bf16x2<false>(src[w]);
    t[2 * w + 1] = e4m3x2_to_bf16x2<true>(src[w]);
  }
  lo = u32x4{__builtin_bit_cast(uint32_t, t[0]), __builtin_bit_cast(uint32_t, t[1]),
             __builtin_bit_cast(uint32_t, t[2]), __builtin_bit_cast(uint32_t, t[3])};
  hi = u32x4{__builtin_bit_cast(uint32_t, t[4]), __builtin_bit_cast(uint32_t, t[5]),
             __builtin_bit_cast(uint32_t, t[6]), __builtin_bit_cast(uint32_t, t[7])};
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- MFMA / LDS
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr));
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = xor_max(v, m);
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
  return v;
}
// max / sum of lane l and lane l ^ 32 in one v_permlane32_swap (no LDS round trip)
__device__ __forceinline__ float half_swap_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_min(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// 2^x on v_exp_f32 directly (no denormal-range fix-up; 2^-inf = 0)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = xor_sum(v, m);
  return v;
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------- balanced schedule geometry
// The page streams of all (request, KV head) units are laid end to end in a
// virtual page space in which every unit u = b*Hkv + g is preceded by A
// placeholder pages standing for the fixed cost of starting a segment (page
// list, query rows, pipeline fill): unit u occupies [start(u), start(u) + A +
// npg_b) and its real pages begin at real(u) = start(u) + A.  Workgroup w owns
// the virtual range [w*TV/W, (w+1)*TV/W); the real pages of one unit inside
// it form a segment, so a workgroup that has to start several segments gets
// correspondingly fewer pages.  Page v belongs to owner(v) = ((v+1)*W - 1)/TV;
// the owners of a unit are owner(real(u)) .. owner(real(u) + npg - 1), every
// one of them holding at least one of its pages when its range is not empty.
// `pfx` is the page prefix over requests (pfx[b] = pages of requests < b).
// floor(n / d) for 0 <= n < 2^53 and d > 0 by one correctly rounded fp64
// division instead of the long 64-bit integer division sequence: n and d
// convert exactly, and a non-integer quotient lies at least 1/d below the
// next integer, which exceeds half an ulp of the quotient (at most n/d *
// 2^-53), so rounding never carries it up to that integer.
__device__ __forceinline__ int64_t floor_div_nonneg(int64_t n, int64_t d) {
  if (n < (int64_t(1) << 53)) return (int64_t)((double)n / (double)d);
  return n / d;
}

struct StreamGeom {
  const int32_t* pfx;
  int32_t Hkv, A;
  int64_t TV, W;
  __device__ int64_t request_start(int b) const { return (int64_t)Hkv * (pfx[b] + (int64_t)A * b); }
  __device__ int64_t npg(int b) const { return pfx[b + 1] - pfx[b]; }
  __device__ int64_t real(int b, int g) const { return request_start(b) + g * (npg(b) + A) + A; }
  __device__ int64_t owner(int64_t v) const { return floor_div_nonneg((v + 1) * W - 1, TV); }
  __device__ bool owns_any(int64_t w) const { return floor_div_nonneg((w + 1) * TV, W) > floor_div_nonneg(w * TV, W); }
};

// ---------------------------------------------------------------- attention sinks
// A sink logit sigma (natural-log units, the units of the scaled scores) folded
// into a finished row: its weight joins the softmax denominator and carries no
// value, so lse becomes ln(e^lse + e^sigma) and the row's output is multiplied
// by the returned e^(lse_old - lse_new) (0 for a row with no visible key, which
// then reports lse = sigma).  sigma = -inf leaves the row unchanged.
__device__ __forceinline__ float fold_sink(float& lse, float sigma) {
  if (sigma == -INFINITY) return 1.f;
  const float hi = fmaxf(lse, sigma);
  const float lse2 = hi + __logf(__expf(lse - hi) + __expf(sigma - hi));
  const float f = __expf(lse - lse2);
  lse = lse2;
  return f;
}

// ---------------------------------------------------------------- error word
__device__ __forceinline__ void flag_error(int32_t* err_word, int32_t bits) {
  if (err_word) atomicOr(err_word, bits);
}

}  // namespace pkv

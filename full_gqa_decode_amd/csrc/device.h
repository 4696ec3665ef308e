// device.h -- gfx950 device helpers shared by the kernels of libflint.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

constexpr int kHeadDim = 128;  // dims per head
constexpr int kPage = 16;      // tokens per page
constexpr int kGroup = 8;      // query heads per KV head
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Value from lane (lane ^ 8) inside each row of 16 lanes (DPP row_ror:8).
__device__ __forceinline__ float lane_xor8(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// Value of lane l ^ 16 / l ^ 32 paired with lane l's, without LDS: with both
// operands x, v_permlane16_swap returns rows (0,0,2,2) and (1,1,3,3) of x and
// v_permlane32_swap halves (0,0) and (1,1), so the two results of one swap
// are {x[l], x[l^16]} (resp. {x[l], x[l^32]}) in some order on every lane.
// (The two results are copied to scalars before the bit casts: a bit cast of
// an element of the builtin's vector result reads element 0.)
__device__ __forceinline__ void swap16(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ void swap32(float x, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_xor16(float x) {
  float a, b;
  swap16(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float max_xor32(float x) {
  float a, b;
  swap32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor16(float x) {
  float a, b;
  swap16(x, a, b);
  return a + b;
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a, b;
  swap32(x, a, b);
  return a + b;
}

// Within each row of 16 lanes, the value of lane (i + K) mod 16 (DPP row_ror).
template <int K>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + K, 0xF, 0xF, false));
}

// Max / sum over the 64 lanes, result in every lane, without LDS.
__device__ __forceinline__ float wave_max_f32(float x) {
  x = fmaxf(x, row_ror<8>(x));
  x = fmaxf(x, row_ror<4>(x));
  x = fmaxf(x, row_ror<2>(x));
  x = fmaxf(x, row_ror<1>(x));
  return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return sum_xor32(sum_xor16(x));
}

__device__ __forceinline__ float readlane_f32(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// fp64 -> bf16 bits with one rounding: round to odd at fp32 precision (24
// bits, enough guard bits for bf16's 8), then round to nearest even.
__device__ __forceinline__ uint16_t bf16_bits_rne_f64(double x) {
  if (x != x) return 0x7fc0u;
  float f = (float)x;
  const double back = (double)f;
  if (back != x) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(x)) u -= 1u;  // the nearest fp32 toward zero
    f = __uint_as_float(u | 1u);
  }
  return bf16_bits_rne(f);
}

// fp64 -> fp8 E4M3 code (OCP E4M3: bias 7, subnormals, no infinities,
// S.1111.111 NaN): nearest, ties to the even code; |x| >= 448 saturates to
// the largest finite code and NaN gives a NaN code.  Within a binade the
// value is scaled by a power of two (exact) onto the integer grid of
// mantissas and rounded by rint (ties to even), so x is rounded once.
__device__ __forceinline__ uint32_t fp8_e4m3_rne_f64(double x) {
  const uint32_t sign = (__builtin_bit_cast(uint64_t, x) >> 63) ? 0x80u : 0u;
  if (x != x) return sign | 0x7Fu;
  const double a = fabs(x);
  if (a >= 448.0) return sign | 0x7Eu;
  if (a < 0.015625) return sign | (uint32_t)rint(a * 512.0);  // step 2^-9 below 2^-6
  int e;
  (void)frexp(a, &e);                                  // a in [2^(e-1), 2^e)
  const uint32_t m = (uint32_t)rint(ldexp(a, 4 - e));  // 8..16 (16 carries)
  return sign | (uint32_t)(((e + 6) << 3) + (int)m - 8);
}

// Element offset of K element (row, dim) inside the 2048-element bf16 tile of
// one (page, KV head): blocks of 32 dims, each in groups of 8 dims, each group
// holding the 8 dims of every row in turn.  Lane l = gq * 16 + n of a wave
// reads K row n's dims c * 32 + gq * 8 .. + 7 (the score MFMA's A operand for
// block c) as 16 contiguous bytes at c * 1024 + l * 16, so each of the four
// loads reads 1 KiB of contiguous bytes.  (V tiles stay dim-major.)
__device__ __forceinline__ int bf16_k_off(int row, int dim) {
  return (dim >> 5) * 512 + ((dim >> 3) & 3) * 128 + row * 8 + (dim & 7);
}

// Byte offsets of K and V element (row, dim) inside the 2048-byte fp8 tile of
// one (page, KV head).  Lane l = gq * 16 + n of a wave reads 16 contiguous
// bytes at l * 16 and at 1024 + l * 16: for K, dims gq * 32 .. gq * 32 + 31 of
// row n; for V, tokens gq * 4 .. gq * 4 + 3 of dims nb * 16 + n, nb = 0..7,
// one dword per nb.  Each of those loads reads 1 KiB of contiguous bytes.
__device__ __forceinline__ int fp8_k_off(int row, int dim) {
  return ((dim >> 4) & 1) * 1024 + (dim >> 5) * 256 + row * 16 + (dim & 15);
}
__device__ __forceinline__ int fp8_v_off(int row, int dim) {
  return (dim >> 6) * 1024 + ((row >> 2) * 16 + (dim & 15)) * 16 + ((dim >> 4) & 3) * 4 +
         (row & 3);
}

// Four fp8 E4M3 codes (bytes 0..3 of w) -> bf16 values in byte order.  Exact:
// every E4M3 value, subnormals included, is a normal bf16 number.  gfx950's
// scaled conversion with scale 1.
__device__ __forceinline__ bf16x4 fp8x4_to_bf16x4(uint32_t w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

// Sum over the 64 lanes, result in every lane: DPP row_ror 8/4/2/1 leaves
// each 16-lane row's total in all its lanes, then the four row totals are
// read as scalars.  No LDS traffic (a shuffle-based version costs ~6 LDS
// round trips on the critical path of the fused decode prologue).
__device__ __forceinline__ double dpp_ror(double x, int k) {
  const int lo = __builtin_bit_cast(int2, x).x, hi = __builtin_bit_cast(int2, x).y;
  int2 r;
  switch (k) {  // the DPP control must be a constant
    case 8: r = int2{__builtin_amdgcn_update_dpp(0, lo, 0x128, 0xF, 0xF, false),
                     __builtin_amdgcn_update_dpp(0, hi, 0x128, 0xF, 0xF, false)}; break;
    case 4: r = int2{__builtin_amdgcn_update_dpp(0, lo, 0x124, 0xF, 0xF, false),
                     __builtin_amdgcn_update_dpp(0, hi, 0x124, 0xF, 0xF, false)}; break;
    case 2: r = int2{__builtin_amdgcn_update_dpp(0, lo, 0x122, 0xF, 0xF, false),
                     __builtin_amdgcn_update_dpp(0, hi, 0x122, 0xF, 0xF, false)}; break;
    default: r = int2{__builtin_amdgcn_update_dpp(0, lo, 0x121, 0xF, 0xF, false),
                      __builtin_amdgcn_update_dpp(0, hi, 0x121, 0xF, 0xF, false)}; break;
  }
  return __builtin_bit_cast(double, r);
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const int2 v = __builtin_bit_cast(int2, x);
  return __builtin_bit_cast(double, int2{__builtin_amdgcn_readlane(v.x, lane),
                                         __builtin_amdgcn_readlane(v.y, lane)});
}

__device__ __forceinline__ double wave_sum_f64(double x) {
  x += dpp_ror(x, 8);
  x += dpp_ror(x, 4);
  x += dpp_ror(x, 2);
  x += dpp_ror(x, 1);
  return (readlane_f64(x, 0) + readlane_f64(x, 16)) + (readlane_f64(x, 32) + readlane_f64(x, 48));
}

// cos/sin of pos * theta^(-2i/128), in fp64 with a two-part 2*pi reduction,
// accurate to ~1e-16 for every position up to the 262,144-token context.
__device__ __forceinline__ void rope_cos_sin(int pos, int i, float theta, double* c, double* s) {
  const double inv_freq = exp2(-(2.0 * i / kHeadDim) * log2((double)theta));
  const double ang = (double)pos * inv_freq;
  const double two_pi_hi = 6.283185307179586;       // 2*pi rounded to fp64
  const double two_pi_lo = 2.4492935982947064e-16;  // 2*pi - two_pi_hi
  const double k = rint(ang * 0.15915494309189535);  // ang / (2*pi)
  double r = fma(-k, two_pi_hi, ang);
  r = fma(-k, two_pi_lo, r);
  sincos(r, s, c);
}

// Per-head RMSNorm then (optionally) rotate-half RoPE of one 128-dim head,
// one wave64: lane l holds dims l and l+64 (a RoPE pair) in x0, x1; on return
// y0, y1 hold the result.  fp64 throughout; cs/sn are rope_cos_sin(pos, l);
// w0, w1 are the norm weights of dims l and l+64 (passed as values so that a
// caller can request them early).  Used by the stand-alone append and by the
// fused decode step, so both produce bit-identical q, K and V.
__device__ __forceinline__ void norm_rope_head(double x0, double x1, float w0, float w1,
                                               float eps, bool rope, double cs, double sn,
                                               double* y0, double* y1) {
  const double ss = wave_sum_f64(x0 * x0 + x1 * x1);
  const double r = 1.0 / sqrt(ss / kHeadDim + (double)eps);
  double a0 = x0 * r * (double)w0;
  double a1 = x1 * r * (double)w1;
  if (rope) {
    const double r0 = a0 * cs - a1 * sn;
    const double r1 = a1 * cs + a0 * sn;
    a0 = r0;
    a1 = r1;
  }
  *y0 = a0;
  *y1 = a1;
}

}  // namespace flint

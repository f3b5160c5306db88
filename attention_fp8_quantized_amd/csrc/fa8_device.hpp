// Device helpers shared by the fa8attn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa8_internal.hpp"   // kFmt* cache formats

namespace fa8 {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBlockSize = 16;

// ---------------------------------------------------------------------------
// e4m3 encoding (OCP E4M3: bias 7, max 448, S.1111.111 = NaN), written as
// integer operations on the float32 bit pattern so the result is exact:
// round-to-nearest-even, saturation at +-448 (also for +-inf), NaN -> 0x7F
// with the input's sign, sign of zero kept.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;                        // NaN
  } else if (a >= 0x43E00000u) {
    code = 0x7Eu;                        // |y| >= 448 (incl. inf): saturate
  } else if (a < 0x3C800000u) {
    // |y| < 2^-6: subnormal codes m * 2^-9, m = rne(|y| * 2^9) in 0..8
    // (scaling by 2^9 is exact; rintf rounds half to even)
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  } else {
    // normal: keep 3 of the 23 mantissa bits with ties-to-even, then rebias
    // the exponent from 127 to 7; a mantissa carry moves into the exponent
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return code | sign;
}

// ---------------------------------------------------------------------------
// e5m2 encoding (OCP E5M2: bias 15, 2 mantissa bits, max finite 57344), the
// same rules as e4m3: round-to-nearest-even, saturation at +-57344 (also for
// +-inf: the cache never holds an infinity), NaN -> 0x7F with the input's
// sign, sign of zero kept.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e5m2_encode(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;                        // NaN
  } else if (a >= 0x47600000u) {
    code = 0x7Bu;                        // |y| >= 57344 (incl. inf): saturate
  } else if (a < 0x38800000u) {
    // |y| < 2^-14: subnormal codes m * 2^-16, m = rne(|y| * 2^16) in 0..4
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f);
  } else {
    // normal: keep 2 of the 23 mantissa bits with ties-to-even, then rebias
    // the exponent from 127 to 15; a mantissa carry moves into the exponent
    const uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
    code = (r >> 21) - (112u << 2);
  }
  return code | sign;
}

template <int kFmt>
__device__ __forceinline__ uint32_t fp8_encode(float y) {
  static_assert(kFmt == kFmtE4m3 || kFmt == kFmtE5m2, "FP8 format");
  if constexpr (kFmt == kFmtE4m3) return e4m3_encode(y);
  else return e5m2_encode(y);
}

// fp32 -> bf16 bits, round-to-nearest-even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two e4m3 codes (bytes 0,1 of w, or 2,3 when kHi) -> two fp32 values (exact).
template <bool kHi>
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, kHi);
}

// Two e4m3 codes -> packed bf16 pair (exact: bf16 holds every e4m3 value).
template <bool kHi>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHi);
}

// Two e4m3 codes -> packed f16 pair (exact: f16 holds every e4m3 value).
template <bool kHi>
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi);
}

// Two e5m2 codes -> bf16 / f16 pairs (exact: e5m2 is the top byte of an
// f16, and bf16 has more exponent and mantissa bits than e5m2).
template <bool kHi>
__device__ __forceinline__ bf16x2 e5m2x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, kHi);
}

template <bool kHi>
__device__ __forceinline__ f16x2 e5m2x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, kHi);
}

// Format-generic forms of the two widenings above.
template <int kFmt, bool kHi>
__device__ __forceinline__ bf16x2 fp8x2_to_bf16(uint32_t w) {
  if constexpr (kFmt == kFmtE5m2) return e5m2x2_to_bf16<kHi>(w);
  else return e4m3x2_to_bf16<kHi>(w);
}

template <int kFmt, bool kHi>
__device__ __forceinline__ f16x2 fp8x2_to_f16(uint32_t w) {
  if constexpr (kFmt == kFmtE5m2) return e5m2x2_to_f16<kHi>(w);
  else return e4m3x2_to_f16<kHi>(w);
}

// acc + a.x*b.x + a.y*b.y  (products of f16 are exact in fp32)
__device__ __forceinline__ float dot2_f16(f16x2 a, f16x2 b, float acc) {
  return __builtin_amdgcn_fdot2(a, b, acc, false);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) {
  return __builtin_bit_cast(bf16x2, w);
}

// acc + a.x*b.x + a.y*b.y  (products of bf16 are exact in fp32)
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

// ---------------------------------------------------------------------------
// Cross-lane sums over aligned groups of N lanes (N = 1..64).  Steps 1 and 2
// use DPP quad permutes, 4 and 8 the row half-mirror / mirror (after the
// lower steps every lane of a quad / half-row holds the same partial, so a
// mirror pairs each lane with a lane of the other half), 16 and 32 fall back
// to a bpermute shuffle.
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                         0xF, 0xF, false));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// fl32(x / s), the quotient correctly rounded, or the cheap product
// q = fl32(x * r) (r = fl32(1 / s), correctly rounded; s positive and normal)
// wherever q encodes to the same FP8 (kFmt) code.  |q - x/s| <= 2 ulp (r
// carries at most half an ulp of relative error, the product rounding
// another half), so q and the correctly rounded quotient lie in the same FP8
// rounding interval unless q is within a few ulp of one of the format's
// rounding midpoints, or in its subnormal range (whose midpoints sit at other
// bit positions).  Only those elements divide exactly.  NaN and infinities
// pass through the product as through the quotient.
template <int kFmt>
__device__ __forceinline__ float fp8_quotient(float x, float s, float r) {
  // bits below the kept mantissa (3 bits e4m3, 2 bits e5m2), the midpoint
  // pattern there, and the smallest normal value of the FP8 format
  constexpr uint32_t kLow = kFmt == kFmtE5m2 ? 0x1FFFFFu : 0xFFFFFu;
  constexpr uint32_t kMid = kFmt == kFmtE5m2 ? 0x100000u : 0x80000u;
  constexpr uint32_t kMinNormal = kFmt == kFmtE5m2 ? 0x38800000u : 0x3C800000u;  // 2^-14 / 2^-6
  constexpr uint32_t kWin = 16;   // ulp of margin on each side of a midpoint
  float y = x * r;
  const uint32_t a = __float_as_uint(y) & 0x7FFFFFFFu;
  const bool near_mid = (a & kLow) - (kMid - kWin) <= 2 * kWin;
  const bool fp8_subnormal = a - 1u < kMinNormal - 1u;   // 0 < |q| < min normal
  if (near_mid || fp8_subnormal) {
    // an opaque step, so that the compiler keeps this a branch instead of
    // dividing every element and selecting
    float xs = x;
    asm volatile("" : "+v"(xs));
    y = xs / s;
  }
  return y;
}

// Two FP8 codes (kFmt) of y0, y1 in the low 16 bits (y0 in bits 0-7): the
// encoding of fp8_encode (round-to-nearest-even, saturation at the largest
// finite value, +-inf included, NaN -> 0x7F with the input's sign, sign of
// zero kept), done by the packed hardware conversion (nearest-even) on
// values first clamped to the largest finite magnitude; NaN is set apart.
template <int kFmt>
__device__ __forceinline__ uint32_t fp8_encode2(float y0, float y1) {
  constexpr uint32_t kMaxBits = kFmt == kFmtE5m2 ? 0x47600000u : 0x43E00000u;  // 57344 / 448
  const uint32_t b0 = __float_as_uint(y0), b1 = __float_as_uint(y1);
  const uint32_t a0 = b0 & 0x7FFFFFFFu, a1 = b1 & 0x7FFFFFFFu;
  const float c0 = __uint_as_float(min(a0, kMaxBits) | (b0 & 0x80000000u));
  const float c1 = __uint_as_float(min(a1, kMaxBits) | (b1 & 0x80000000u));
  uint32_t w;
  if constexpr (kFmt == kFmtE5m2)
    w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c0, c1, 0, false);
  else
    w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  w &= 0xFFFFu;
  if (a0 > 0x7F800000u) w = (w & 0xFF00u) | 0x7Fu | (b0 >> 24 & 0x80u);
  if (a1 > 0x7F800000u) w = (w & 0x00FFu) | ((0x7Fu | (b1 >> 24 & 0x80u)) << 8);
  return w;
}

// One 16-byte chunk of a cached row from its input elements (fp32 or bf16):
// 16 FP8 codes (kFmt e4m3 or e5m2) of fl32(x / scale) (correctly rounded
// quotient: callers are built without fast-math and with correctly rounded
// division), or 8 bf16 values (kFmtBf16, scale unused).  `elem` indexes the
// input in elements.
template <bool kInBf16, int kFmt>
__device__ __forceinline__ uint4 encode_chunk(const void* src, int64_t elem, float scale) {
  constexpr bool kFp8Cache = kFmt != kFmtBf16;
  constexpr int N = kFp8Cache ? 16 : 8;
  float x[N];
  if constexpr (kInBf16) {
    const uint4* ptr = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + elem);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const uint4 w = ptr[i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[i * 8 + 2 * j] = bf16_lo(ws[j]);
        x[i * 8 + 2 * j + 1] = bf16_hi(ws[j]);
      }
    }
  } else {
    const float4* ptr = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + elem);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const float4 w = ptr[i];
      x[i * 4 + 0] = w.x;
      x[i * 4 + 1] = w.y;
      x[i * 4 + 2] = w.z;
      x[i * 4 + 3] = w.w;
    }
  }
  uint32_t packed[4];
  if constexpr (kFp8Cache) {
    const float rcp = 1.0f / scale;   // correctly rounded, once per chunk
    float y[N];
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = fp8_quotient<kFmt>(x[i], scale, rcp);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      packed[w] = fp8_encode2<kFmt>(y[4 * w], y[4 * w + 1]) |
                  (fp8_encode2<kFmt>(y[4 * w + 2], y[4 * w + 3]) << 16);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) packed[w] = bf16_bits(x[2 * w]) | (bf16_bits(x[2 * w + 1]) << 16);
  }
  return make_uint4(packed[0], packed[1], packed[2], packed[3]);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

}  // namespace fa8

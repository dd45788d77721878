// Device helpers of the fp8 casts with a bf16 scale (row-wise and
// tensor-wise; gist "FP8 linear triton with row-wise scaling",
// quantize_fp8_rowwise): the scale from an amax, and eight elements at a
// time from bf16 to e4m3fn under that scale.
//
// scale = amax / 448 formed in binary32 and rounded to bf16 (0x7FC0 for a
// NaN amax); code = binary32(x) / scale converted to e4m3fn, nearest-even,
// not saturated (above 464 and +-Inf -> NaN); the sign bit of every code is
// the sign bit of x.
//
// The quotient.  For a normal, finite scale s, r = 1/s is formed once
// (correctly rounded); per element q0 = x * r, the exact residual e = x - q0
// * s by one fma, and q = q0 + e * r by another.  With r correctly rounded
// and q0 within an ulp of x / s this is the correctly rounded binary32
// quotient (Markstein's theorem): three operations instead of a full IEEE
// division sequence.  For such a scale |x / s| <= 448 * (1 + 2^-8) < 464, so
// no code overflows.  Zero, subnormal, Inf and NaN scales (uniform over the
// elements that share them) take IEEE division and an explicit overflow
// test.  The e4m3 rounding is gfx950's scaled convert with scale 1, fed
// magnitudes no larger than 448.
#pragma once

#include "mx_device.h"

namespace mx {

constexpr float kE4m3Max = 448.0f;
constexpr float kE4m3Overflow = 464.0f;   // midpoint of 448 and 480 (no finite code)

struct Fp8Scale {
  uint32_t bits;  // bf16 bits of the scale
  float s;        // the scale as binary32 (exact)
  float r;        // 1 / s, correctly rounded (fast path)
  bool fast;      // s normal and finite
};

// bf16 bits of the scale for an amax given as magnitude bits (NaN > Inf >
// finite).
__device__ __forceinline__ uint32_t fp8_scale_bits(uint32_t amax) {
  if (amax > kInfBits)
    return 0x7FC0u;
  if (amax == kInfBits)
    return kInfBits;
  // binary32 quotient (IEEE division), then nearest-even to the top 16 bits:
  // adding 0x7FFF plus the kept LSB carries exactly when the dropped half is
  // above one half, or equal to it with an odd LSB.
  const uint32_t u = __float_as_uint(__uint_as_float(amax << 16) / kE4m3Max);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Everything the element rule needs from the scale's bf16 bits.
__device__ __forceinline__ Fp8Scale fp8_scale_of_bits(uint32_t bits) {
  Fp8Scale p;
  p.bits = bits;
  p.s = __uint_as_float(bits << 16);
  const uint32_t ef = bits & kInfBits;
  p.fast = ef != 0 && ef != kInfBits;
  p.r = 1.0f / p.s;
  return p;
}

__device__ __forceinline__ Fp8Scale fp8_scale(uint32_t amax) { return fp8_scale_of_bits(fp8_scale_bits(amax)); }

// Correctly rounded |x| / s for a normal finite s with r = RN(1 / s).
__device__ __forceinline__ float div_fast(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(e, r, q0);
}

// Magnitude code of a quotient when the scale is not normal and finite: NaN
// and anything past 464 (Inf included) has no finite code; (448, 464] rounds
// to 448.
__device__ __forceinline__ float slow_clamp(float q, bool& nan) {
  nan = !(q <= kE4m3Overflow);
  return __builtin_fminf(q, kE4m3Max);
}

// Sign bits of four bf16 values (two packed pairs) in the code byte positions.
__device__ __forceinline__ uint32_t signs4(uint32_t x01, uint32_t x23) {
  return __builtin_amdgcn_perm(x23, x01, 0x07050301u) & 0x80808080u;
}

// Eight bf16 values (one 16-byte chunk) -> eight e4m3fn bytes.
template <bool FAST>
__device__ __forceinline__ uint2 quant8(const uint4& d, const Fp8Scale& p) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float m[4];
    bool nan[4] = {false, false, false, false};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t v = w[2 * h + k] & kMagMask2;
      const float lo = __uint_as_float(v << 16);
      const float hi = __uint_as_float(v & 0xFFFF0000u);
      if (FAST) {
        m[2 * k] = div_fast(lo, p.s, p.r);
        m[2 * k + 1] = div_fast(hi, p.s, p.r);
      } else {
        m[2 * k] = slow_clamp(lo / p.s, nan[2 * k]);
        m[2 * k + 1] = slow_clamp(hi / p.s, nan[2 * k + 1]);
      }
    }
    i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((i16x2){0, 0}, m[0], m[1], 1.0f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, m[2], m[3], 1.0f, true);
    uint32_t c = as_u32(r);
    if (!FAST) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (nan[k])
          c |= 0x7Fu << (8 * k);
    }
    out[h] = c | signs4(w[2 * h], w[2 * h + 1]);
  }
  return make_uint2(out[0], out[1]);
}

// One bf16 value -> its e4m3fn byte (ragged and unaligned paths).
__device__ __forceinline__ uint32_t quant1(uint32_t x, const Fp8Scale& p) {
  const uint4 d = make_uint4(x & 0xFFFFu, 0, 0, 0);
  return (p.fast ? quant8<true>(d, p) : quant8<false>(d, p)).x & 0xFFu;
}

__device__ __forceinline__ uint32_t chunk_amax(const uint4& d) {
  return max2(max2(mag2(d.x), mag2(d.y)), max2(mag2(d.z), mag2(d.w)));
}

// Max over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
    v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

}  // namespace mx

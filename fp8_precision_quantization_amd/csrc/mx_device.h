// Device helpers shared by the libmxcast kernels (gfx950 only).
//
// bf16 data is handled as raw 16-bit patterns, two per 32-bit register.  The
// block amax is an unsigned max of the magnitude bits (sign cleared): for
// IEEE formats the magnitude bits order like the values, and NaN > +Inf >
// every finite value, so the max also flags non-finite blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kMagMask2 = 0x7FFF7FFFu;  // clears both sign bits
constexpr uint32_t kInfBits = 0x7F80u;         // bf16 +Inf magnitude

__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ i16x2 as_i16x2(uint32_t v) { return __builtin_bit_cast(i16x2, v); }
__device__ __forceinline__ uint32_t as_u32(i16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Workgroup barrier that orders LDS only.  __syncthreads() is a full
// workgroup fence: it would also wait for every outstanding global load and
// store of the wave, which the kernels here want to keep in flight across
// the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Raw buffer resource over [base, base + bytes) for buffer loads and stores
// whose row offset sits in a scalar register (no per-lane address math).
// The third descriptor word is the gfx950 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Store of 16 bytes that, across the lanes of one instruction, make up whole
// 128-byte lines: non-temporal.  Stores that cover only part of a line stay
// ordinary (cached) instead: non-temporal ones there keep the L2 from merging
// the partial lines that neighbouring lanes and workgroups write, which
// multiplies HBM writes.
__device__ __forceinline__ void store_line_nt(uint8_t* p, const uint4& v) {
  __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// Per-half unsigned max of two packed 16-bit pairs (v_pk_max_u16).
__device__ __forceinline__ uint32_t max2(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_max(as_u16x2(a), as_u16x2(b)));
}

// Packed magnitude bits of two bf16 values.
__device__ __forceinline__ uint32_t mag2(uint32_t x) { return x & kMagMask2; }

// Clamp the magnitudes of two bf16 values to the limit t2 (same 15-bit limit
// in both halves, sign clear), keeping each sign.  Negative patterns are
// >= 0x8000 as unsigned and < 0 as signed, so an unsigned min against
// (limit | sign) clamps the negatives and a signed min against the limit
// clamps the positives; neither touches the other sign.
__device__ __forceinline__ uint32_t clamp_mag2(uint32_t x, uint32_t t2, uint32_t t2_neg) {
  uint32_t a = as_u32(__builtin_elementwise_min(as_u16x2(x), as_u16x2(t2_neg)));
  return as_u32(__builtin_elementwise_min(as_i16x2(a), as_i16x2(t2)));
}

// Four bf16 values (two packed pairs) -> four e4m3 bytes, x / 2^(scale
// exponent) rounded to nearest-even.  gfx950's scaled convert takes the scale
// as a binary32 whose exponent field is used as is, so an e8m0 byte shifted
// into that field (byte << 23) is the block scale, byte 0 (2^-127) included.
// The instruction does not saturate: the caller clamps beforehand.
__device__ __forceinline__ uint32_t cvt4_e4m3(uint32_t x01, uint32_t x23, float scale) {
  i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((i16x2){0, 0}, __builtin_bit_cast(bf16x2, x01),
                                                      scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2, x23), scale, true);
  return as_u32(r);
}

// DPP cross-lane moves inside groups of four lanes.
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {  // lanes 1,0,3,2
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {  // lanes 2,3,0,1
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}
// Lane i of each group of eight reads lane 7 - i (the other quad).
__device__ __forceinline__ uint32_t half_row_mirror(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
}

// Everything a block's amax decides.
//   kind 0: finite block.  byte = max(E - 8, 0) with E the amax exponent
//           field, which is floor(log2 amax) - 8 + 127 clamped at the bottom
//           (an all-zero or denormal amax lands on byte 0).  Elements are
//           clamped to 448 * 2^e, whose bf16 pattern is ((byte + 8) << 7) |
//           0x60, before the convert, which is exact for every bf16 value.
//   kind 1: amax = +Inf (no NaN).  e = 127, byte 254; finite elements scale
//           to below 2 and need no clamp; +-Inf convert to NaN and are
//           rewritten as +-448 afterwards.
//   kind 2: a NaN in the block.  byte 0xFF; every element becomes NaN with
//           its own sign.
struct BlockParams {
  uint32_t t2;      // magnitude limit, both halves
  uint32_t t2_neg;  // t2 with both sign bits set
  float scale;      // binary32 with the e8m0 byte in its exponent field
  uint32_t byte;    // e8m0 scale byte
  uint32_t kind;
};

template <bool SPECIAL>
__device__ __forceinline__ BlockParams block_params(uint32_t amax_bits) {
  BlockParams p;
  uint32_t t;
  if (!SPECIAL || amax_bits < kInfBits) {
    uint32_t e_field = amax_bits >> 7;
    p.byte = e_field > 8 ? e_field - 8 : 0;
    t = ((p.byte + 8) << 7) | 0x60;
    p.kind = 0;
  } else if (amax_bits == kInfBits) {
    p.byte = 254;
    t = kInfBits;
    p.kind = 1;
  } else {
    p.byte = 0xFF;
    t = kInfBits;
    p.kind = 2;
  }
  p.t2 = t | (t << 16);
  p.t2_neg = p.t2 | 0x80008000u;
  p.scale = __uint_as_float((p.byte & 0xFF) << 23);
  return p;
}

// Four elements of one block -> four e4m3 bytes.
template <bool SPECIAL>
__device__ __forceinline__ uint32_t quant4(uint32_t x01, uint32_t x23, const BlockParams& p) {
  uint32_t r = cvt4_e4m3(clamp_mag2(x01, p.t2, p.t2_neg), clamp_mag2(x23, p.t2, p.t2_neg), p.scale);
  if (SPECIAL) {
    if (p.kind == 2) {
      uint32_t signs = ((x01 >> 8) & 0x80u) | ((x01 >> 16) & 0x8000u) | ((x23 << 8) & 0x800000u) |
                       (x23 & 0x80000000u);
      r = 0x7F7F7F7Fu | signs;
    } else if (p.kind == 1) {
      // NaN codes here come only from +-Inf inputs: 0x7F -> 0x7E, 0xFF -> 0xFE.
      r -= (((r & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) >> 7;
    }
  }
  return r;
}

}  // namespace mx

// Device-side OCP E4M3FN quantization for gfx950.
//
// Rule (FP8-RL summary page, "Prerequisites / FP8 quantization format": one scale
// per block, W_hat = round(W / scale), E4M3 range about +-448):
//   scale = fl32(amax / range) (1 when amax == 0);
//   code  = E4M3FN value nearest to the EXACT real quotient x / scale, ties to the
//           even code, saturating at +-448, sign of -0 kept.
//
// An fp32 quotient (or x * (1/scale)) is not the exact quotient: it can land on a
// rounding midpoint the exact quotient only approaches, and then round the wrong
// way.  The encoder therefore works in three steps per element:
//   1. t = |x| * r with r = 1/scale: within a few fp32 ulps of |x|/scale, so it
//      identifies the rounding interval up to the one midpoint `mid` nearest t;
//   2. the sign of fma(-mid, scale, |x|) = |x| - mid*scale, computed with one
//      rounding and therefore with its exact sign, says on which side of `mid` the
//      exact quotient lies (zero means an exact tie);
//   3. `mid` is nudged one fp32 ulp to that side (not at all on a tie) and the
//      hardware round-to-nearest-even conversion produces the code.  On a tie the
//      conversion's own ties-to-even rule picks the even code.
// `mid` comes from the fp32 bits of t: clearing all but three mantissa bits gives
// the E4M3 value below t and setting the next bit gives the midpoint above it.  For
// quotients below 2^-6 (E4M3 subnormals, spacing 2^-9) t is first shifted by 2^-6
// into the binade [2^-6, 2^-5), whose spacing is the same 2^-9, and shifted back; the
// shift is folded into the FMA that forms t.  Which side of 2^-6 takes the shift is
// decided by comparing |x| with lim = fl((2^-6 - 2^-20) * scale): the shifted path is
// exact for t < 2^-6 - 2^-29 (t + 2^-6 stays below 2^-5) and the plain path for
// t >= 2^-6 - 2^-11 (the nearest E4M3 midpoint below is 2^-6 - 2^-10), and the few-ulp
// fuzz of the comparison stays well inside that overlap.
//
// The residual needs scale * mid to be representable down to its last bit: that
// holds when scale >= 2^-116.  Smaller scales (data around 1e-33 and below) take a
// slow path that multiplies both x and scale by 2^64 first, which changes neither
// the quotient nor any rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr float kE4M3Max = 448.0f;
constexpr float kSubnormalSwitch = 0x1.ffffcp-7f;  // 2^-6 - 2^-20
constexpr float kTinyScale = 0x1p-116f;

// bf16 bit patterns packed two per dword -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Scale from the amax: fl32(amax / range), 1 for amax == 0.
__device__ __forceinline__ float scale_from_amax(float amax, float range) {
  return amax == 0.0f ? 1.0f : amax / range;
}

// Power-of-two (UE8M0) scale variant: the smallest 2^e with range * 2^e >= amax, e in
// the E8M0 exponent range [-127, 127]; 1 for amax == 0.  range * 2^e is exact in binary32
// for every e reached from a bf16 amax, so the comparisons decide exactly.
__device__ __forceinline__ float scale_pow2_from_amax(float amax, float range) {
  if (amax == 0.0f) return 1.0f;
  const int biased = (int)((__float_as_uint(amax) >> 23) & 0xffu);
  int e = (biased ? biased - 127 : -127) - 8;  // within a few steps of the answer
  while (range * __builtin_ldexpf(1.0f, e) < amax) ++e;
  while (range * __builtin_ldexpf(1.0f, e - 1) >= amax) --e;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return __builtin_ldexpf(1.0f, e);
}

template <bool POW2>
__device__ __forceinline__ float block_scale(float amax, float range) {
  if constexpr (POW2) {
    return scale_pow2_from_amax(amax, range);
  } else {
    return scale_from_amax(amax, range);
  }
}

struct Quantizer {
  float s;    // scale as used in the residual test (possibly x 2^64)
  float r;    // 1 / s
  float lim;  // |x| below this takes the subnormal shift
  float xm;   // factor applied to x (1 or 2^64)
};

__device__ __forceinline__ Quantizer make_quantizer(float scale) {
  Quantizer q;
  if (scale < kTinyScale) {
    q.s = scale * 0x1p64f;
    q.xm = 0x1p64f;
  } else {
    q.s = scale;
    q.xm = 1.0f;
  }
  q.r = 1.0f / q.s;
  q.lim = kSubnormalSwitch * q.s;
  return q;
}

// fp32 bits with the mantissa cut to 3 bits and the next bit set: the midpoint above
// the E4M3 value below (one bitfield insert).
__device__ __forceinline__ uint32_t keep3_set_half(uint32_t bits) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(0xfff00000u), "v"(bits), "v"(0x00080000u));
  return r;
}

// -1, 0 or +1 by the sign of a float's bit pattern read as an integer (+0 gives 0).
__device__ __forceinline__ int sign_of(float v) {
  int r;
  asm("v_med3_i32 %0, %1, -1, 1" : "=v"(r) : "v"(__float_as_int(v)));
  return r;
}

// The fp32 value whose round-to-nearest-even E4M3 conversion is the code of x/s.
// `ax` is |x| (already multiplied by the tiny-scale factor when that path is used).
// SAT: clamp the nudged value to 448 (needed only when x/s may exceed 464, i.e. with
// a stored scale; with scale = amax/448 the quotient never exceeds 449.6).
template <bool SAT>
__device__ __forceinline__ float nudged_magnitude(float ax, const Quantizer& q) {
  const float off = (ax < q.lim) ? 0x1p-6f : 0.0f;
  const float tt = fminf(__builtin_fmaf(ax, q.r, off), kE4M3Max);
  const float mid = __uint_as_float(keep3_set_half(__float_as_uint(tt))) - off;
  const float res = __builtin_fmaf(-mid, q.s, ax);
  float v = __uint_as_float(__float_as_uint(mid) + (uint32_t)sign_of(res));
  if (SAT) v = fminf(v, kE4M3Max);
  return v;
}

template <bool SAT>
__device__ __forceinline__ float nudged(float x, const Quantizer& q, bool tiny) {
  float ax = fabsf(x);
  if (tiny) ax *= q.xm;
  const float v = nudged_magnitude<SAT>(ax, q);
  return __builtin_copysignf(v, x);  // v >= 0: takes x's sign, -0 included
}

// Four fp32 values (already nudged) -> four packed E4M3FN bytes, element 0 lowest.
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Quantize 8 bf16 (one uint4 = 4 dwords) into 8 codes (uint2).
template <bool SAT>
__device__ __forceinline__ uint2 quant8(uint4 w, const Quantizer& q, bool tiny) {
  uint2 o;
  o.x = cvt4(nudged<SAT>(bf16_lo(w.x), q, tiny), nudged<SAT>(bf16_hi(w.x), q, tiny),
             nudged<SAT>(bf16_lo(w.y), q, tiny), nudged<SAT>(bf16_hi(w.y), q, tiny));
  o.y = cvt4(nudged<SAT>(bf16_lo(w.z), q, tiny), nudged<SAT>(bf16_hi(w.z), q, tiny),
             nudged<SAT>(bf16_lo(w.w), q, tiny), nudged<SAT>(bf16_hi(w.w), q, tiny));
  return o;
}

// Quantize 16 bf16 (two uint4) into 16 codes (uint4); the tiny-scale path is taken
// only when the scale demands it (uniform for a block, rare for a group).
template <bool SAT>
__device__ __forceinline__ uint4 quant16(uint4 a, uint4 b, const Quantizer& q) {
  uint2 lo, hi;
  if (q.xm == 1.0f) {
    lo = quant8<SAT>(a, q, false);
    hi = quant8<SAT>(b, q, false);
  } else {
    lo = quant8<SAT>(a, q, true);
    hi = quant8<SAT>(b, q, true);
  }
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Largest |x| of 16 bf16 values as magnitude bits (bf16 magnitudes order like
// unsigned integers): packed 16-bit maxima of the sign-cleared pairs.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 mag2(uint32_t w) { return __builtin_bit_cast(u16x2, w & 0x7fff7fffu); }
__device__ __forceinline__ uint32_t absmax16(uint4 a, uint4 b) {
  u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(mag2(a.x), mag2(a.y)),
                                      __builtin_elementwise_max(mag2(a.z), mag2(a.w)));
  m = __builtin_elementwise_max(m, __builtin_elementwise_max(__builtin_elementwise_max(mag2(b.x), mag2(b.y)),
                                                             __builtin_elementwise_max(mag2(b.z), mag2(b.w))));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Largest |x| of 8 bf16 values as magnitude bits.
__device__ __forceinline__ uint32_t absmax8(uint4 a) {
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(mag2(a.x), mag2(a.y)),
                                            __builtin_elementwise_max(mag2(a.z), mag2(a.w)));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Max over groups of 8 consecutive lanes (DPP: quad swaps then half-row mirror).
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));  // [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));  // [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false)); // half mirror
  return v;
}

// Max over the whole wave (64 lanes).
__device__ __forceinline__ uint32_t max_over_wave(uint32_t v) {
  v = max_over_8_lanes(v);
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false)); // row mirror
  // combine the four rows of 16 lanes
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h) { return __uint_as_float(h << 16); }

// 16-byte global accesses.  The streaming (non-temporal) forms keep data touched once
// out of the caches; the plain forms let it stay for a consumer that follows.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
typedef unsigned int u32x2e __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8_stream(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2e{v.x, v.y}, reinterpret_cast<u32x2e*>(p));
}
__device__ __forceinline__ uint4 load_plain(const void* p) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_plain(void* p, uint4 v) {
  *reinterpret_cast<u32x4*>(p) = u32x4{v.x, v.y, v.z, v.w};
}

}  // namespace fp8q

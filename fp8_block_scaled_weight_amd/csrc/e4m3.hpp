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
// into the binade [2^-6, 2^-5), whose spacing is the same 2^-9, and shifted back.
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
// Largest float below 2^-6: quotients below it use the subnormal shift.
constexpr float kSubnormalLimit = 0x1.fffffep-7f;
constexpr float kTinyScale = 0x1p-116f;

// bf16 bit patterns packed two per dword -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// |x| as an order-preserving integer for the packed pair (bf16 magnitude bits).
__device__ __forceinline__ uint32_t bf16x2_absmax(uint32_t acc, uint32_t w) {
  uint32_t lo = w & 0x7fffu;
  uint32_t hi = (w >> 16) & 0x7fffu;
  return max(acc, max(lo, hi));
}

// Scale from the amax magnitude bits (bf16): fl32(amax / range), 1 for amax == 0.
__device__ __forceinline__ float scale_from_amax(float amax, float range) {
  return amax == 0.0f ? 1.0f : amax / range;
}

struct Quantizer {
  float s;    // scale as used in the residual test (possibly x 2^64)
  float r;    // 1 / s
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
  return q;
}

// The fp32 value whose round-to-nearest-even E4M3 conversion is the code of x/s.
// `ax` is |x| (already multiplied by the tiny-scale factor when that path is used).
// SAT: clamp the nudged value to 448 (needed only when x/s may exceed 464, i.e. with
// a stored scale; with scale = amax/448 the quotient never exceeds 449.6).
template <bool SAT>
__device__ __forceinline__ float nudged_magnitude(float ax, float s, float r) {
  float t = fminf(ax * r, kE4M3Max);
  float off = (t < kSubnormalLimit) ? 0x1p-6f : 0.0f;
  float tt = t + off;
  float mid = __uint_as_float((__float_as_uint(tt) & 0xfff00000u) | 0x00080000u) - off;
  float res = __builtin_fmaf(-mid, s, ax);
  int side = min(max((int)__float_as_uint(res), -1), 1);  // sign of res: -1, 0, +1
  float v = __uint_as_float(__float_as_uint(mid) + (uint32_t)side);
  if (SAT) v = fminf(v, kE4M3Max);
  return v;
}

template <bool SAT>
__device__ __forceinline__ float nudged(float x, const Quantizer& q, bool tiny) {
  float ax = fabsf(x);
  if (tiny) ax *= q.xm;
  float v = nudged_magnitude<SAT>(ax, q.s, q.r);
  return __uint_as_float(__float_as_uint(v) | (__float_as_uint(x) & 0x80000000u));
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

__device__ __forceinline__ uint32_t absmax16(uint4 a, uint4 b) {
  uint32_t m = 0;
  m = bf16x2_absmax(m, a.x);
  m = bf16x2_absmax(m, a.y);
  m = bf16x2_absmax(m, a.z);
  m = bf16x2_absmax(m, a.w);
  m = bf16x2_absmax(m, b.x);
  m = bf16x2_absmax(m, b.y);
  m = bf16x2_absmax(m, b.z);
  m = bf16x2_absmax(m, b.w);
  return m;
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

// 16-byte streaming (non-temporal) global accesses: data touched once is not kept.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}

}  // namespace fp8q

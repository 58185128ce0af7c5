// SwiGLU fused with the 1x128 E4M3 quantization of its output, per group of 128 values
// held by 8 consecutive lanes (16 each).  Shared by the standalone kernel and the
// epilogue of the MoE fc1 GEMM, so that both produce the same bits.
#pragma once

#include "e4m3.hpp"

namespace fp8q {

// ----------------------------------------------------------------------------
// SwiGLU + 1x128 quantization.  h = [gate | up], bf16 [m, 2n]; a = silu(gate) * up.
// The value is defined in fp64, g / (1 + exp(-g)) * u, far inside fp32 precision, so the
// E4M3 encoding is its one rounding.  Per row and 128-column group: amax = max |a|
// (exact), scale = fl32(fl64(amax / 448)) (1 for amax 0), code = the E4M3 value nearest
// the fp64 quotient a / scale (ties to even, saturating).
//
// Fast path.  Each value is first formed in fp32 (relative error below 2^-20: exp(-g)
// within about 2.5 ulps, one rounding each for 1 + e, the reciprocal and two products),
// and the fp64 value is formed only where the fp32 one cannot decide:
//   - inputs outside the range where that bound holds (gate <= -80, where expf
//     overflows; |gate| or |up| >= 2^60; |a| below 2^-100 unless a is an exact zero);
//   - the group maximum: every value within 2^-14 of the fp32 maximum is recomputed in
//     fp64, so amax is the fp64 maximum;
//   - codes: the fp32 quotient is moved by 2^-15 both ways; if both give one code, the
//     fp64 quotient (within 2^-19 of it) gives that code too, since rounding is monotone;
//     otherwise the code comes from the fp64 quotient.  Groups with a scale below
//     2^-100 take the fp64 path throughout.
// An fp64 quotient is rounded to fp32 with round-to-odd (truncate, then set the last bit
// if anything was dropped), which keeps enough information for the hardware's
// round-to-nearest-even conversion to give the nearest code of the fp64 value.
// Same lane mapping as the activation quantizer: 8 lanes per group, 16 values each.
// ----------------------------------------------------------------------------
__device__ __forceinline__ double silu_times_up(double g, double u) {
#pragma clang fp contract(off)
  return g / (1.0 + exp(-g)) * u;
}

// exp(x) for x < 80: 2^(x log2 e) with the exponent carried as an fp32 head ph plus its
// remainder pl (fma-exact product remainder and the low part of log2 e); the hardware
// 2^ph (about 1 ulp) is corrected by the first-order factor 1 + pl ln 2 (|pl| <= 2^-17,
// so the dropped second-order term is below 2^-35).  Very negative x gives 0.
__device__ __forceinline__ float exp_lt80(float x) {
  constexpr float kL2eHi = 0x1.715476p+0f;    // log2(e) rounded to fp32
  constexpr float kL2eLo = 0x1.4ae0c0p-26f;   // log2(e) - kL2eHi, rounded
  constexpr float kLn2 = 0x1.62e430p-1f;
  const float ph = x * kL2eHi;
  const float pl = __builtin_fmaf(x, kL2eHi, -ph) + x * kL2eLo;
  return __builtin_amdgcn_exp2f(ph) * __builtin_fmaf(pl, kLn2, 1.0f);
}

__device__ __forceinline__ float silu_times_up_f32(float g, float u) {
#pragma clang fp contract(off)
  return g * __builtin_amdgcn_rcpf(1.0f + exp_lt80(-g)) * u;
}

__device__ __forceinline__ float round_to_odd_f32(double u) {
  const double au = fabs(u);
  uint32_t b = __float_as_uint((float)au);
  if ((double)__uint_as_float(b) > au) b -= 1u;           // toward zero
  if ((double)__uint_as_float(b) != au) b |= 1u;          // sticky
  return __builtin_copysignf(fminf(__uint_as_float(b), kE4M3Max), (float)u);
}

__device__ __forceinline__ double max_over_8_lanes_f64(double v) {
  v = fmax(v, __shfl_xor(v, 1));
  v = fmax(v, __shfl_xor(v, 2));
  v = fmax(v, __shfl_xor(v, 4));
  return v;
}

// gate and up of value i (0..15) of this lane, selected without dynamic register indexing
__device__ __forceinline__ double swiglu_at(const uint32_t (&gw)[8], const uint32_t (&uw)[8], int i) {
  uint32_t gword = gw[0], uword = uw[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    gword = ((i >> 1) == j) ? gw[j] : gword;
    uword = ((i >> 1) == j) ? uw[j] : uword;
  }
  const float g = (i & 1) ? bf16_hi(gword) : bf16_lo(gword);
  const float u = (i & 1) ? bf16_hi(uword) : bf16_lo(uword);
  return silu_times_up((double)g, (double)u);
}

// Power-of-two (UE8M0) scale of an fp64 group maximum: the smallest 2^e with
// 448 * 2^e >= amax (exact fp64 comparisons), e limited to the E8M0 range [-127, 127];
// 1 for amax == 0.  The start is within a few steps of the answer.
__device__ __forceinline__ float scale_pow2_from_amax_f64(double amax) {
  if (amax == 0.0) return 1.0f;
  const int biased = (int)((__double_as_longlong(amax) >> 52) & 0x7ff);
  int e = (biased ? biased - 1023 : -1074) - 8;
  while ((double)kE4M3Max * ldexp(1.0, e) < amax) ++e;
  while ((double)kE4M3Max * ldexp(1.0, e - 1) >= amax) --e;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return __builtin_ldexpf(1.0f, e);
}

constexpr float kSwigluCodeSlack = 0x1p-15f;   // relative move of the fp32 quotient
constexpr double kSwigluMaxSlack = 0x1p-14;     // values this close to the maximum are recomputed

// One lane's part of a group: gw/uw hold its 16 gate and 16 up values (bf16 pairs, value
// i in half i & 1 of word i >> 1); the 8 lanes of a group (lane & 7 = 0..7, aligned)
// call together, dead lanes included, since the group maximum is reduced by shuffles.
// Returns false for a dead lane; otherwise sets the group's scale and the lane's 16
// codes (o[w] byte e = value 4w + e).  POW2: the group's scale is the power of two above
// (the codes then follow from the same exact quotient rule).
template <bool POW2 = false>
__device__ __forceinline__ bool swiglu_quant16(const uint32_t (&gw)[8], const uint32_t (&uw)[8], bool live,
                                               uint32_t (&o)[4], float& scale) {
  // fp32 values, and the values that need fp64 from the start
  float a32[16];
  uint32_t slow = 0;
  float m32 = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float gv = (i & 1) ? bf16_hi(gw[i >> 1]) : bf16_lo(gw[i >> 1]);
    const float uv = (i & 1) ? bf16_hi(uw[i >> 1]) : bf16_lo(uw[i >> 1]);
    const float a = silu_times_up_f32(gv, uv);
    const bool exact_zero = (gv == 0.0f) || (uv == 0.0f);
    const bool ok = exact_zero || (gv > -80.0f && fabsf(gv) < 0x1p60f && fabsf(uv) < 0x1p60f && fabsf(a) >= 0x1p-100f);
    slow |= ok ? 0u : (1u << i);
    a32[i] = ok ? a : 0.0f;
    m32 = fmaxf(m32, fabsf(a32[i]));
  }

  // amax in fp64: the fp64 values of the slow ones and of every value near the maximum
  double approx = (double)m32, amax = 0.0;
  for (uint32_t t = slow; t; t &= t - 1) {
    const double a = fabs(swiglu_at(gw, uw, __builtin_ctz(t)));
    approx = fmax(approx, a);
    amax = fmax(amax, a);
  }
  approx = max_over_8_lanes_f64(approx);
  if (approx > 0.0) {
    const float thr = (float)(approx * (1.0 - kSwigluMaxSlack));
    uint32_t cand = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) cand |= (fabsf(a32[i]) >= thr) ? (1u << i) : 0u;
    cand &= ~slow;
    for (; cand; cand &= cand - 1) amax = fmax(amax, fabs(swiglu_at(gw, uw, __builtin_ctz(cand))));
  }
  amax = max_over_8_lanes_f64(amax);
  if (!live) return false;
  scale = POW2 ? scale_pow2_from_amax_f64(amax) : (amax == 0.0) ? 1.0f : (float)(amax / (double)kE4M3Max);

  // codes: fp32 quotient moved both ways; the fp64 quotient where they disagree
#pragma unroll
  for (int w = 0; w < 4; ++w) o[w] = 0u;
  uint32_t need = 0xffffu;
  if (scale >= 0x1p-100f) {
    need = slow;
    const float r32 = 1.0f / scale;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = a32[4 * w + e] * r32;
        const float av = fabsf(v);
        lo[e] = __builtin_copysignf(fminf(av * (1.0f - kSwigluCodeSlack), kE4M3Max), v);
        hi[e] = __builtin_copysignf(fminf(av * (1.0f + kSwigluCodeSlack), kE4M3Max), v);
      }
      const uint32_t cl = cvt4(lo[0], lo[1], lo[2], lo[3]);
      const uint32_t diff = cl ^ cvt4(hi[0], hi[1], hi[2], hi[3]);
      o[w] = cl;
#pragma unroll
      for (int e = 0; e < 4; ++e) need |= ((diff >> (8 * e)) & 0xffu) ? (1u << (4 * w + e)) : 0u;
    }
  }
  const double sd = (double)scale;
  for (; need; need &= need - 1) {
    const int i = __builtin_ctz(need);
    const uint32_t c = cvt4(round_to_odd_f32(swiglu_at(gw, uw, i) / sd), 0.0f, 0.0f, 0.0f) & 0xffu;
    const int sh = 8 * (i & 3);
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = ((i >> 2) == w) ? ((o[w] & ~(0xffu << sh)) | (c << sh)) : o[w];
  }
  return true;
}

}  // namespace fp8q

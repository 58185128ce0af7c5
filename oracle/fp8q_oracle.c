/*
 * fp8q oracle: a plain, slow, obviously correct CPU implementation of the
 * FP8 rollout hot path (blockwise weight quantization, per-token-group
 * activation quantization, block-scaled W8A8 GEMM dense and grouped, FP8 KV
 * cache quantize-on-write with per-step scale recalibration).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) shares no code, header, table or constant generator with it.
 *
 * Sources (page title, then section):
 *   [FP8-RL] "FP8-RL: A Practical and Stable Low-Precision Stack for LLM
 *            Reinforcement Learning" (paper summary page)
 *       - "Prerequisites / FP8 quantization format": E4M3 (4 exponent bits,
 *         3 mantissa bits, range about +-448); 128x128 blockwise weight
 *         quantization with one scale per block and W_hat = round(W/scale).
 *       - "Method step details", step 1: weights quantized at sync, activations
 *         quantized dynamically on every forward; step 3: FP8 KV cache whose
 *         K/V scales are recalibrated before each RL step's rollout.
 *       - "Experimental results": FP32 scale factors (not power-of-two).
 *   [Rounding] "Where rounding happens matters" (BF16 rounding-location page),
 *       section on what rounding-location mismatch is: BF16 has 8 significant
 *       bits; keep fused math in FP32 and round once at the output.
 *   [1T-RL] "1T-parameter RL on 100 GPUs", section 3.4: paged KV cache in
 *       fixed-size blocks, K and V each quantized to FP8 separately.
 *   [R3] MoE routing-replay page ("Rollout Routing Replay", section 4, and the
 *       cost analysis, section 5): each token's top-8 expert indices are kept
 *       as int16 and tokens are dispatched to those recorded experts.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - E4M3 is OCP E4M3FN: bias 7, max 448 (0x7E), subnormals m*2^-9, NaN 0x7F.
 *   - scale = fl32(amax / 448) (IEEE binary32 division); the page writes
 *     scale = max|W_block|, and 448 maps the block maximum onto the E4M3 max.
 *     An all-zero block/group gets scale 1.
 *   - q = the E4M3FN value nearest the exact real quotient x/scale, ties to
 *     the even code, saturating at +-448, sign of -0 kept (0x80).
 *   - activations: 1x128 groups along K; scale (m, g) stored at s[g*ld_s+m].
 *   - GEMM: exact dequantize, fp64 accumulation, fp64 output.
 *   - KV: one fp32 scale per tensor (K, V) per call; amax over the tokens the
 *     call writes (slot >= 0).
 *   - Power-of-two (UE8M0) scale variant, the alternative the "Experimental
 *     results" ablation compares with FP32 scales: scale = the smallest power
 *     of two 2^e with 448 * 2^e >= amax (the block maximum still fits the E4M3
 *     range), e limited to the E8M0 exponent range [-127, 127]; 1 for amax 0.
 *     The quotient x / 2^e is then exact and only the E4M3 rounding remains.
 *   - SwiGLU before MoE fc2 ([Rounding], SwiGLU fusion region): silu(gate)*up in
 *     fp64, quantized once per 1x128 group with the rule above (scale
 *     fl32(fl64(amax / 448))).
 *   - FP8 decode attention: the query quantized with its own recalibrated scale,
 *     FP8 x FP8 scores, softmax and the V sum in fp64 (see below).
 *   - MoE dispatch and combine ([R3]) are integer gathers and an fp64 sum;
 *     they are written in numpy in __init__.py.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * Every entry point returns 0 on success, -1 on non-finite input, -2 on a bad
 * shape.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define E4M3_MAX 448.0

/* ---- BF16 and E4M3FN decoding, straight from the format definitions ---- */

static float bf16_to_float(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16; /* bf16 is the top half of binary32 */
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* OCP E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent field 0 encodes subnormals m * 2^-9.  0x7F / 0xFF are NaN. */
double oracle_e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sign ? -v : v;
}

/* The 127 non-negative finite values, codes 0x00..0x7E, increasing. */
static double g_pos[127];
static int g_pos_ready = 0;

static void init_table(void) {
  if (g_pos_ready) return;
#pragma omp critical(fp8q_oracle_table)
  {
    if (!g_pos_ready) {
      for (int c = 0; c < 127; ++c) g_pos[c] = oracle_e4m3_decode((uint8_t)c);
      g_pos_ready = 1;
    }
  }
}

/* Nearest E4M3FN code to u: clamp |u| to 448, find the largest table value
 * <= |u| by bisection, then compare |u| with the midpoint to the next value
 * (exact in fp64); a tie picks the code with an even last bit.  The sign comes
 * from u's sign bit, so -0 and small negatives give 0x80. */
uint8_t oracle_e4m3_encode(double u) {
  init_table();
  int neg = signbit(u) ? 1 : 0;
  double a = fabs(u);
  if (a > E4M3_MAX) a = E4M3_MAX;
  int lo = 0, hi = 126;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (g_pos[mid] <= a)
      lo = mid;
    else
      hi = mid - 1;
  }
  int c = lo;
  if (c < 126) {
    double midpoint = 0.5 * (g_pos[c] + g_pos[c + 1]);
    if (a > midpoint || (a == midpoint && (c & 1))) c = c + 1;
  }
  return (uint8_t)((neg ? 0x80 : 0x00) | c);
}

/* scale = fl32(amax / range), an IEEE binary32 division; 1 for amax == 0. */
float oracle_scale(float amax, float range) {
  if (amax == 0.0f) return 1.0f;
  return amax / range;
}

/* Power-of-two (UE8M0) scale [FP8-RL, "Experimental results", scale-format
 * ablation]: 2^e for the smallest integer e with range * 2^e >= amax, found by
 * exact comparisons (range * 2^e is exact in binary32 here), then limited to
 * [-127, 127]; 1 for amax == 0.  2^-127 is a binary32 subnormal, still exact. */
float oracle_scale_ue8m0(float amax, float range) {
  if (amax == 0.0f) return 1.0f;
  int e = ilogbf(amax) - ilogbf(range);
  while ((double)range * ldexp(1.0, e) < (double)amax) ++e;
  while ((double)range * ldexp(1.0, e - 1) >= (double)amax) --e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return ldexpf(1.0f, e);
}

typedef float (*scale_rule_fn)(float amax, float range);

/* One element: the fp64 quotient x/s decides every E4M3 rounding exactly as
 * the real quotient would (x has 8 and s 24 significant bits, so x/s is either
 * exactly a midpoint or at least ~2^-29 relative away from it). */
uint8_t oracle_quantize_value(float x, float s) {
  return oracle_e4m3_encode((double)x / (double)s);
}

/* ---- a1: 128x128 blockwise weight quantization [FP8-RL, FP8 format] ---- */
static int quant_weight_rule(const uint16_t* w, int64_t n, int64_t k, int64_t ld_w,
                             uint8_t* q, int64_t ld_q, float* s, scale_rule_fn rule) {
  if (n < 0 || k < 0 || n % 128 || k % 128 || ld_w < k || ld_q < k) return -2;
  int64_t nb = n / 128, kb = k / 128;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
  for (int64_t bi = 0; bi < nb; ++bi) {
    for (int64_t bj = 0; bj < kb; ++bj) {
      float amax = 0.0f;
      for (int64_t r = 0; r < 128; ++r) {
        for (int64_t c = 0; c < 128; ++c) {
          float x = bf16_to_float(w[(bi * 128 + r) * ld_w + bj * 128 + c]);
          if (!isfinite(x)) bad = 1;
          float a = fabsf(x);
          if (a > amax) amax = a;
        }
      }
      float sc = rule(amax, (float)E4M3_MAX);
      s[bi * kb + bj] = sc;
      for (int64_t r = 0; r < 128; ++r) {
        for (int64_t c = 0; c < 128; ++c) {
          float x = bf16_to_float(w[(bi * 128 + r) * ld_w + bj * 128 + c]);
          q[(bi * 128 + r) * ld_q + bj * 128 + c] = oracle_quantize_value(x, sc);
        }
      }
    }
  }
  return bad ? -1 : 0;
}

int oracle_quant_weight_blk128(const uint16_t* w, int64_t n, int64_t k, int64_t ld_w,
                               uint8_t* q, int64_t ld_q, float* s) {
  return quant_weight_rule(w, n, k, ld_w, q, ld_q, s, oracle_scale);
}

int oracle_quant_weight_blk128_ue8m0(const uint16_t* w, int64_t n, int64_t k, int64_t ld_w,
                                     uint8_t* q, int64_t ld_q, float* s) {
  return quant_weight_rule(w, n, k, ld_w, q, ld_q, s, oracle_scale_ue8m0);
}

/* ---- a2: dynamic 1x128 activation quantization [FP8-RL, step 1] ----
 * Scale of row m, group g is stored at s[g*ld_s + m]. */
static int quant_act_rule(const uint16_t* x, int64_t m, int64_t k, int64_t ld_x,
                          uint8_t* q, int64_t ld_q, float* s, int64_t ld_s, scale_rule_fn rule) {
  if (m < 0 || k < 0 || k % 128 || ld_x < k || ld_q < k || ld_s < m) return -2;
  int64_t groups = k / 128;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
  for (int64_t row = 0; row < m; ++row) {
    for (int64_t g = 0; g < groups; ++g) {
      float amax = 0.0f;
      for (int64_t c = 0; c < 128; ++c) {
        float v = bf16_to_float(x[row * ld_x + g * 128 + c]);
        if (!isfinite(v)) bad = 1;
        float a = fabsf(v);
        if (a > amax) amax = a;
      }
      float sc = rule(amax, (float)E4M3_MAX);
      s[g * ld_s + row] = sc;
      for (int64_t c = 0; c < 128; ++c) {
        float v = bf16_to_float(x[row * ld_x + g * 128 + c]);
        q[row * ld_q + g * 128 + c] = oracle_quantize_value(v, sc);
      }
    }
  }
  return bad ? -1 : 0;
}

int oracle_quant_act_g128(const uint16_t* x, int64_t m, int64_t k, int64_t ld_x,
                          uint8_t* q, int64_t ld_q, float* s, int64_t ld_s) {
  return quant_act_rule(x, m, k, ld_x, q, ld_q, s, ld_s, oracle_scale);
}

int oracle_quant_act_g128_ue8m0(const uint16_t* x, int64_t m, int64_t k, int64_t ld_x,
                                uint8_t* q, int64_t ld_q, float* s, int64_t ld_s) {
  return quant_act_rule(x, m, k, ld_x, q, ld_q, s, ld_s, oracle_scale_ue8m0);
}

/* ---- SwiGLU fused with the 1x128 quantization between MoE fc1 and fc2 ----
 * [Rounding], the SwiGLU fusion region: the fused form keeps SiLU's result
 * unrounded and multiplies it by the up projection before the one rounding;
 * [FP8-RL] step 1: fc2's input is quantized dynamically in 1x128 groups.
 * h is the bf16 fc1 output [m, 2*n]: gate = columns [0, n), up = [n, 2n).
 * Reading: a = g / (1 + exp(-g)) * u evaluated in fp64 (finer than fp32, so the
 * E4M3 encoding is the only rounding that matters); per row and 128-column
 * group, amax = max |a| (exact), s = fl32(fl64(amax / 448)), 1 for amax 0;
 * code = E4M3 nearest of the fp64 quotient a / s.  Precondition: amax / 448
 * fits binary32.  amax_out (may be NULL) receives the fp64 amax of group g of
 * row r at amax_out[g*m + r], so that a caller can see how close a scale was
 * to an fp32 rounding boundary. */
static double silu_times_up(double g, double u) { return g / (1.0 + exp(-g)) * u; }

/* The power-of-two rule of oracle_scale_ue8m0 for an fp64 amax: 2^e for the smallest
 * integer e with range * 2^e >= amax (exact fp64 comparisons), limited to [-127, 127];
 * 1 for amax == 0. */
static float scale_ue8m0_f64(double amax, double range) {
  if (amax == 0.0) return 1.0f;
  int e = ilogb(amax) - ilogb(range);
  while (range * ldexp(1.0, e) < amax) ++e;
  while (range * ldexp(1.0, e - 1) >= amax) --e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return ldexpf(1.0f, e);
}

static int swiglu_quant_rule(const uint16_t* h, int64_t m, int64_t n, int64_t ld_h, uint8_t* q,
                             int64_t ld_q, float* s, int64_t ld_s, double* amax_out, int ue8m0) {
  if (m < 0 || n < 0 || n % 128 || ld_h < 2 * n || ld_q < n || ld_s < m) return -2;
  int64_t groups = n / 128;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
  for (int64_t row = 0; row < m; ++row) {
    for (int64_t g = 0; g < groups; ++g) {
      double a[128];
      double amax = 0.0;
      for (int64_t c = 0; c < 128; ++c) {
        float gv = bf16_to_float(h[row * ld_h + g * 128 + c]);
        float uv = bf16_to_float(h[row * ld_h + n + g * 128 + c]);
        if (!isfinite(gv) || !isfinite(uv)) bad = 1;
        a[c] = silu_times_up((double)gv, (double)uv);
        if (fabs(a[c]) > amax) amax = fabs(a[c]);
      }
      float sc = ue8m0 ? scale_ue8m0_f64(amax, E4M3_MAX) : (amax == 0.0) ? 1.0f : (float)(amax / E4M3_MAX);
      s[g * ld_s + row] = sc;
      if (amax_out) amax_out[g * m + row] = amax;
      for (int64_t c = 0; c < 128; ++c) q[row * ld_q + g * 128 + c] = oracle_e4m3_encode(a[c] / (double)sc);
    }
  }
  return bad ? -1 : 0;
}

int oracle_swiglu_quant_g128(const uint16_t* h, int64_t m, int64_t n, int64_t ld_h, uint8_t* q,
                             int64_t ld_q, float* s, int64_t ld_s, double* amax_out) {
  return swiglu_quant_rule(h, m, n, ld_h, q, ld_q, s, ld_s, amax_out, 0);
}

/* The same with the power-of-two (UE8M0) scale of the fp64 group maximum
 * [FP8-RL, "Experimental results", scale-format ablation]; the code is then the E4M3
 * nearest of the exact quotient a / 2^e. */
int oracle_swiglu_quant_g128_ue8m0(const uint16_t* h, int64_t m, int64_t n, int64_t ld_h, uint8_t* q,
                                   int64_t ld_q, float* s, int64_t ld_s, double* amax_out) {
  return swiglu_quant_rule(h, m, n, ld_h, q, ld_q, s, ld_s, amax_out, 1);
}

/* SiLU(g) * u of one element, as above (exposed for the tests' pins). */
double oracle_silu_times_up(double g, double u) { return silu_times_up(g, u); }

/* ---- FP8 paged decode attention [FP8-RL, "Method step details" step 3 (per-step
 * recalibration of the Q/K/V scales) and "Experimental results" (full FP8: linear,
 * KV cache and attention); 1T-RL 3.4 (paged cache in fixed blocks)] ----
 * Reading: the query is quantized to E4M3 with its own per-layer scale (the same rule
 * as K and V: scale = fl32(amax / range) over the call's queries when recalibrating),
 * scores are the FP8 x FP8 products s = sm_scale * q_scale * k_scale * sum_d
 * dec(cq[d]) * dec(ck[t][d]), p = softmax over the sequence's L tokens, and
 * out[d] = v_scale * sum_t p_t * dec(cv[t][d]).  Everything after the codes in fp64.
 * Query head h reads KV head h / (hq / hkv).  Token t of sequence b sits in page
 * block_table[b*ld_bt + t / page_size], slot t % page_size; caches are
 * [page][slot][hkv][128] bytes.  q: bf16 [seqs][hq][128] rows with pitch ld_q per
 * sequence; out: fp64 [seqs][hq][128]. */
int oracle_q_scale(const uint16_t* q, int64_t ld_q, int32_t seqs, int32_t hq, float range, float* q_scale) {
  float amax = 0.0f;
  for (int32_t b = 0; b < seqs; ++b)
    for (int64_t i = 0; i < (int64_t)hq * 128; ++i) {
      float v = bf16_to_float(q[b * ld_q + i]);
      if (!isfinite(v)) return -1;
      if (fabsf(v) > amax) amax = fabsf(v);
    }
  *q_scale = oracle_scale(amax, range);
  return 0;
}

int oracle_paged_decode_attention(const uint16_t* q, int64_t ld_q, const uint8_t* kc, const uint8_t* vc,
                                  const int32_t* block_table, int64_t ld_bt, const int32_t* seq_lens, int32_t seqs,
                                  int32_t hq, int32_t hkv, int32_t page_size, float q_scale, float k_scale,
                                  float v_scale, double sm_scale, double* out) {
  if (seqs < 0 || hq < 1 || hkv < 1 || hq % hkv || page_size < 1) return -2;
  const int32_t group = hq / hkv;
  int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : bad)
  for (int32_t b = 0; b < seqs; ++b) {
    for (int32_t h = 0; h < hq; ++h) {
      const int32_t L = seq_lens[b];
      const int32_t g = h / group;
      double* o = out + ((int64_t)b * hq + h) * 128;
      for (int d = 0; d < 128; ++d) o[d] = 0.0;
      if (L <= 0) continue;
      double cq[128];
      for (int d = 0; d < 128; ++d) {
        float x = bf16_to_float(q[b * ld_q + (int64_t)h * 128 + d]);
        if (!isfinite(x)) bad = 1;
        cq[d] = oracle_e4m3_decode(oracle_quantize_value(x, q_scale));
      }
      double* sc = (double*)malloc(sizeof(double) * (size_t)L);
      const double f = sm_scale * (double)q_scale * (double)k_scale;
      double mx = -INFINITY;
      for (int32_t t = 0; t < L; ++t) {
        const int64_t page = block_table[(int64_t)b * ld_bt + t / page_size];
        const uint8_t* k = kc + ((page * page_size + t % page_size) * hkv + g) * 128;
        double dot = 0.0;
        for (int d = 0; d < 128; ++d) dot += cq[d] * oracle_e4m3_decode(k[d]);
        sc[t] = f * dot;
        if (sc[t] > mx) mx = sc[t];
      }
      double z = 0.0;
      for (int32_t t = 0; t < L; ++t) {
        sc[t] = exp(sc[t] - mx);
        z += sc[t];
      }
      for (int32_t t = 0; t < L; ++t) {
        const int64_t page = block_table[(int64_t)b * ld_bt + t / page_size];
        const uint8_t* v = vc + ((page * page_size + t % page_size) * hkv + g) * 128;
        const double p = sc[t] / z;
        for (int d = 0; d < 128; ++d) o[d] += p * oracle_e4m3_decode(v[d]);
      }
      for (int d = 0; d < 128; ++d) o[d] *= (double)v_scale;
      free(sc);
    }
  }
  return bad ? -1 : 0;
}

/* ---- a3: block-scaled W8A8 GEMM [FP8-RL, step 1; Rounding] ----
 * y[i][j] = sum_kb (sa[kb][i] * sb[j/128][kb]) * sum_{t in kb} dec(a[i][t]) dec(b[j][t])
 * All in fp64: every decoded value is an integer multiple of 2^-9 below 2^9,
 * so each 128-term block sum is exact; the scale product of two binary32
 * numbers is exact; only the outer sum rounds (about 1e-16 relative). */
int oracle_gemm_w8a8(const uint8_t* a, int64_t ld_a, const float* as, int64_t ld_as,
                     const uint8_t* b, int64_t ld_b, const float* bs,
                     double* y, int64_t ld_y, int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k < 0 || k % 128 || n % 128 || ld_a < k || ld_b < k || ld_y < n ||
      ld_as < m)
    return -2;
  init_table();
  int64_t kblocks = k / 128;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      double acc = 0.0;
      for (int64_t kb = 0; kb < kblocks; ++kb) {
        double partial = 0.0;
        for (int64_t t = kb * 128; t < kb * 128 + 128; ++t)
          partial += oracle_e4m3_decode(a[i * ld_a + t]) * oracle_e4m3_decode(b[j * ld_b + t]);
        double scale = (double)as[kb * ld_as + i] * (double)bs[(j / 128) * kblocks + kb];
        acc += scale * partial;
      }
      y[i * ld_y + j] = acc;
    }
  }
  return 0;
}

/* ---- a4: MoE grouped block-scaled GEMM [FP8-RL, step 1 and results] ----
 * Rows [off[g], off[g+1]) of a use expert g's weight b[g] ([n][k]) and scales
 * bs[g] ([n/128][k/128]). */
int oracle_grouped_gemm_w8a8(const uint8_t* a, int64_t ld_a, const float* as, int64_t ld_as,
                             const uint8_t* b, const float* bs, const int32_t* off,
                             int32_t groups, double* y, int64_t ld_y, int64_t n, int64_t k) {
  if (groups < 1 || n % 128 || k % 128 || ld_a < k || ld_y < n) return -2;
  for (int32_t g = 0; g < groups; ++g)
    if (off[g + 1] < off[g] || off[0] != 0) return -2;
  if (ld_as < off[groups]) return -2;
  init_table();
  int64_t kblocks = k / 128;
  for (int32_t g = 0; g < groups; ++g) {
    const uint8_t* bg = b + (int64_t)g * n * k;
    const float* bsg = bs + (int64_t)g * (n / 128) * kblocks;
    int64_t r0 = off[g], r1 = off[g + 1];
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = r0; i < r1; ++i) {
      for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int64_t kb = 0; kb < kblocks; ++kb) {
          double partial = 0.0;
          for (int64_t t = kb * 128; t < kb * 128 + 128; ++t)
            partial += oracle_e4m3_decode(a[i * ld_a + t]) * oracle_e4m3_decode(bg[j * k + t]);
          double scale = (double)as[kb * ld_as + i] * (double)bsg[(j / 128) * kblocks + kb];
          acc += scale * partial;
        }
        y[i * ld_y + j] = acc;
      }
    }
  }
  return 0;
}

/* ---- a5 + a6: FP8 KV cache quantize-on-write with recalibration ----
 * [FP8-RL, step 3]: before each RL step's rollout the K/V scales are
 * recomputed from the data; [1T-RL, 3.4]: paged cache, K and V separately.
 * Token t with slot = slot_mapping[t] >= 0 is written to cache position
 * [slot / page_size][slot % page_size][head][dim], i.e. byte offset
 * slot * heads * head_dim.  With recalibrate != 0 the scales are first set to
 * fl32(amax / range) over every element this call writes (1 when amax is 0);
 * otherwise *k_scale and *v_scale are used as given.  Unwritten cache bytes are
 * left untouched. */
int oracle_kv_quant(const uint16_t* kx, int64_t ld_k, const uint16_t* vx, int64_t ld_v,
                    int64_t tokens, int32_t heads, int32_t head_dim,
                    const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                    int32_t page_size, int64_t num_pages, float* k_scale, float* v_scale,
                    float range, int recalibrate) {
  int64_t row = (int64_t)heads * head_dim;
  if (tokens < 0 || heads < 1 || head_dim < 1 || page_size < 1 || ld_k < row || ld_v < row)
    return -2;
  for (int64_t t = 0; t < tokens; ++t)
    if (slot_mapping[t] >= num_pages * page_size) return -2;
  int bad = 0;
  if (recalibrate) {
    float ak = 0.0f, av = 0.0f;
    for (int64_t t = 0; t < tokens; ++t) {
      if (slot_mapping[t] < 0) continue;
      for (int64_t e = 0; e < row; ++e) {
        float xk = bf16_to_float(kx[t * ld_k + e]);
        float xv = bf16_to_float(vx[t * ld_v + e]);
        if (!isfinite(xk) || !isfinite(xv)) bad = 1;
        if (fabsf(xk) > ak) ak = fabsf(xk);
        if (fabsf(xv) > av) av = fabsf(xv);
      }
    }
    *k_scale = oracle_scale(ak, range);
    *v_scale = oracle_scale(av, range);
  }
  float sk = *k_scale, sv = *v_scale;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    for (int64_t e = 0; e < row; ++e) {
      k_cache[slot * row + e] = oracle_quantize_value(bf16_to_float(kx[t * ld_k + e]), sk);
      v_cache[slot * row + e] = oracle_quantize_value(bf16_to_float(vx[t * ld_v + e]), sv);
    }
  }
  return bad ? -1 : 0;
}

/* ---- a5 alone: the recalibrated K/V scales of a call, without writing the cache ----
 * [FP8-RL, step 3]: scale = fl32(amax / range) over every element the call writes
 * (tokens with slot >= 0), 1 when that amax is 0.  Same definition as the recalibrating
 * branch of oracle_kv_quant, for inputs too large to encode in full on the host. */
int oracle_kv_scales(const uint16_t* kx, int64_t ld_k, const uint16_t* vx, int64_t ld_v, int64_t tokens,
                     int64_t row, const int64_t* slot_mapping, float range, float* k_scale, float* v_scale) {
  if (tokens < 0 || row < 1 || ld_k < row || ld_v < row) return -2;
  float ak = 0.0f, av = 0.0f;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(max : ak, av) reduction(| : bad)
  for (int64_t t = 0; t < tokens; ++t) {
    if (slot_mapping[t] < 0) continue;
    for (int64_t e = 0; e < row; ++e) {
      float xk = bf16_to_float(kx[t * ld_k + e]);
      float xv = bf16_to_float(vx[t * ld_v + e]);
      if (!isfinite(xk) || !isfinite(xv)) bad = 1;
      if (fabsf(xk) > ak) ak = fabsf(xk);
      if (fabsf(xv) > av) av = fabsf(xv);
    }
  }
  *k_scale = oracle_scale(ak, range);
  *v_scale = oracle_scale(av, range);
  return bad ? -1 : 0;
}

/* Number of OpenMP threads the oracle uses (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * fp8q.h: C ABI of libfp8q, the FP8 rollout hot path on AMD Instinct MI355X (gfx950).
 *
 * The library implements, as hand-written HIP kernels for one GPU:
 *   - 128x128 blockwise E4M3 weight quantization, run at every RL weight sync;
 *   - dynamic 1x128 per-token-group activation quantization, run on every forward;
 *   - the block-scaled W8A8 GEMM that consumes both, dense and MoE-grouped;
 *   - FP8 KV-cache quantize-on-write with per-step K/V scale recalibration;
 *   - around the grouped GEMM: MoE dispatch by recorded expert ids, SwiGLU fused with
 *     fc2's 1x128 quantization (standalone, or in fc1's epilogue), and the weighted
 *     combine;
 *   - FP8 paged decode attention over that cache, with the query scale recalibrated
 *     per step.
 *
 * Sources (page title, then section):
 *   [FP8-RL]   "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
 *              Learning" (paper summary page): "Prerequisites / FP8 quantization format"
 *              (E4M3 with range about +-448; one scale per 128x128 weight block,
 *              W_hat = round(W / scale)); "Method step details" step 1 (W8A8 linears:
 *              weights quantized statically at sync, activations dynamically per
 *              forward; q/k/v/o, gate/up/down and MoE fc1/fc2 quantized, embedding,
 *              norms and lm_head not), step 2 (three-stage weight sync: init, sync with
 *              blockwise quantization, inference), step 3 (FP8 KV cache, scales
 *              recalibrated before every RL step's rollout); "Experimental results"
 *              (FP32 scale factors preferred over power-of-two ones).
 *   [Rounding] "Where rounding happens matters" (BF16 rounding-location page), section
 *              on rounding-location mismatch: keep fused arithmetic in FP32 and round
 *              to BF16 once, at the output.
 *   [1T-RL]    "1T-parameter RL on 100 GPUs", section 3.4: paged KV cache in fixed
 *              blocks; K and V each quantized to FP8 separately.
 *   [R3]       MoE routing-replay page: "Rollout Routing Replay" (section 4: the rollout
 *              records each token's expert indices and tokens are dispatched to the
 *              recorded experts) and the cost analysis (section 5: 8 int16 indices per
 *              token and layer).
 *
 * Number formats.  FP8 codes are OCP E4M3FN bytes (bias 7, max +-448 = 0x7E/0xFE,
 * subnormals m * 2^-9, NaN 0x7F/0xFF never produced).  BF16 inputs/outputs are
 * 16-bit brain floats.  Scales are IEEE binary32.
 *
 * Quantization rule (every quantizer in this header):
 *   amax  = max |x| over the block, group or call (exact);
 *   scale = fl32(amax / range), an IEEE binary32 division; 1.0 if amax == 0;
 *           range = 448 except where a call takes it as an argument;
 *   code  = the E4M3FN value nearest to the exact real quotient x / scale, ties to
 *           the even code, saturating to +-448; the sign of -0 is kept (0x80).
 * The results are unique: codes and scales are bit-exact and deterministic.
 *
 * Power-of-two (UE8M0) scale variant, the entry points named *_ue8m0 [FP8-RL,
 * "Experimental results": the scale-format ablation compares FP32 scales with UE8M0
 * (power-of-two) ones]: scale = the smallest power of two 2^e with 448 * 2^e >= amax,
 * e limited to the E8M0 exponent range [-127, 127] (2^-127 is a binary32 subnormal);
 * 1.0 if amax == 0.  Codes follow the same rule (the quotient x / 2^e is exact).  Scales
 * are still stored as binary32 values, in the same layouts.
 *
 * Conventions for every call.
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns every
 *     buffer.  The library allocates no memory and keeps no state besides the
 *     per-thread error string.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.  Every
 *     call validates its arguments on the host, enqueues its kernels on `stream` and
 *     returns without synchronizing.  Stream order is the only ordering.
 *   - Leading dimensions (`ld_*`) count elements of the buffer's type (bytes for FP8,
 *     2-byte units for BF16, floats for scales).
 *   - On any error nothing is enqueued and the returned status says why;
 *     fp8q_last_error() gives a readable detail.  Device-side faults surface at the
 *     caller's next synchronization.
 *   - Preconditions not checked (undefined behaviour if violated): inputs are finite;
 *     outputs do not overlap inputs or each other; group offsets are nondecreasing
 *     with offsets[0] = 0 and offsets[G] = total_m; every KV slot is below
 *     num_pages * page_size; and the per-call preconditions stated below.
 *   - Debug mode: with the environment variable FP8Q_DEBUG=1 (read at every call) a call
 *     also checks those preconditions before it enqueues anything, and returns
 *     FP8Q_ERR_PRECONDITION, with the offending element in fp8q_last_error(), if one
 *     fails.  It checks that outputs overlap no input or other output (byte extents);
 *     and, after synchronizing `stream` and copying the data to the host: bf16 and fp32
 *     inputs are finite, FP8 operands of the GEMMs hold no NaN code (0x7F/0xFF), GEMM
 *     scales are finite (powers of two for *_ue8m0), group offsets and KV slots are in
 *     range, and the attention call's lengths, page ids and stored scales are valid.
 *     Not checked even then: the FP8 codes of the KV caches, whose size makes a host
 *     copy impractical, and the combine's row indices against the rows of y, which the
 *     call is not told.  After the launch a debug-mode call synchronizes `stream`, so a
 *     device fault is reported (FP8Q_ERR_LAUNCH) by the call that caused it.  Debug
 *     mode cannot run on a stream under graph capture (FP8Q_ERR_UNSUPPORTED).
 *   - Calls are thread-safe.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_ABI_VERSION 1

typedef enum fp8q_status {
  FP8Q_OK = 0,
  FP8Q_ERR_NULL = 1,        /* a required pointer is NULL */
  FP8Q_ERR_SHAPE = 2,       /* negative size, size not a multiple of 128 where required,
                               count/num_groups < 1, head_dim != 128, page_size < 1 */
  FP8Q_ERR_STRIDE = 3,      /* a leading dimension is smaller than the row length */
  FP8Q_ERR_ALIGN = 4,       /* a data pointer or row pitch is not 16-byte aligned */
  FP8Q_ERR_LAUNCH = 5,      /* the HIP runtime refused a launch (with FP8Q_DEBUG=1 also:
                               the kernel faulted, or a debug read of device data failed) */
  FP8Q_ERR_UNSUPPORTED = 6, /* no gfx950 device is current; with FP8Q_DEBUG=1 also: the
                               stream is being captured */
  FP8Q_ERR_PRECONDITION = 7 /* FP8Q_DEBUG=1 only: a precondition listed above is violated */
} fp8q_status;

/* Static string naming a status code. */
const char* fp8q_status_string(fp8q_status s);
/* Detail of the last failure on the calling thread ("" if none).  Valid until the
 * thread's next fp8q call. */
const char* fp8q_last_error(void);
/* FP8Q_ABI_VERSION of the loaded library. */
int fp8q_abi_version(void);

/* ------------------------------------------------------------------------------
 * Blockwise weight quantization  [FP8-RL, "Prerequisites / FP8 quantization format";
 * "Method step details" steps 1-2]
 *
 * One descriptor per nn.Linear weight, or per stack of expert weights viewed as one
 * [E*n, k] matrix.  For every 128x128 block (bi, bj) of w (blocks aligned at (0,0)):
 *   s[bi * (k/128) + bj] = scale of the block;  q[r * ld_q + c] = code of w[r * ld_w + c].
 *   w: bf16 [n, k] row-major, row pitch ld_w elements (ld_w >= k, ld_w % 8 == 0).
 *   q: e4m3fn [n, k] row-major, row pitch ld_q bytes (ld_q >= k, ld_q % 16 == 0).
 *   s: fp32 [n/128][k/128] row-major, contiguous.
 *   n % 128 == 0 and k % 128 == 0 (else FP8Q_ERR_SHAPE); n == 0 or k == 0 is a no-op
 *   for that descriptor.  w and q 16-byte aligned (else FP8Q_ERR_ALIGN).
 * descs is a HOST array of `count` descriptors (count >= 1), read during the call only:
 * one call quantizes a whole weight sync (e.g. all linears of all layers).
 * ---------------------------------------------------------------------------- */
typedef struct fp8q_weight_desc {
  const void* w;  /* bf16 [n][ld_w] (device) */
  void* q;        /* e4m3fn [n][ld_q] (device) */
  float* s;       /* fp32 [n/128][k/128] (device) */
  int64_t n, k;   /* rows (output features), columns (input features) */
  int64_t ld_w;   /* elements */
  int64_t ld_q;   /* bytes */
} fp8q_weight_desc;

fp8q_status fp8q_quant_weight_blk128(const fp8q_weight_desc* descs /* host */, int32_t count,
                                     void* stream);

/* The same with power-of-two (UE8M0) scales; arguments, layouts and errors as above. */
fp8q_status fp8q_quant_weight_blk128_ue8m0(const fp8q_weight_desc* descs /* host */,
                                           int32_t count, void* stream);

/* ------------------------------------------------------------------------------
 * Dynamic per-token-group activation quantization  [FP8-RL, "Method step details"
 * step 1: activations quantized dynamically on every forward]
 *
 * For row r < m and group g < k/128 (128 consecutive columns):
 *   s[g * ld_s + r] = scale of x[r, 128g .. 128g+127];
 *   q[r * ld_q + c] = code of x[r * ld_x + c].
 *   x: bf16 [m, k], ld_x >= k, ld_x % 8 == 0; q: e4m3fn [m, k], ld_q >= k, ld_q % 16 == 0;
 *   s: fp32 [k/128][ld_s], ld_s >= m (scales of one group are contiguous over rows, the
 *   layout the GEMM reads).  k % 128 == 0.  m == 0 is a no-op.
 * ---------------------------------------------------------------------------- */
fp8q_status fp8q_quant_act_g128(const void* x, int64_t m, int64_t k, int64_t ld_x, void* q,
                                int64_t ld_q, float* s, int64_t ld_s, void* stream);

/* The same with power-of-two (UE8M0) scales; arguments, layouts and errors as above. */
fp8q_status fp8q_quant_act_g128_ue8m0(const void* x, int64_t m, int64_t k, int64_t ld_x, void* q,
                                      int64_t ld_q, float* s, int64_t ld_s, void* stream);

/* ------------------------------------------------------------------------------
 * Block-scaled W8A8 GEMM  [FP8-RL, "Method step details" step 1; Rounding]
 *
 *   y[r, j] = bf16_rne( sum_{kb < k/128} a_s[kb * ld_as + r] * b_s[(j/128) * (k/128) + kb]
 *                        * sum_{t in block kb} dec(a[r, t]) * dec(b[j, t]) )
 * The per-block scale product is applied to each 128-wide partial sum in the fp32
 * accumulator; the result is rounded to bf16 once (round to nearest even).
 *   a:   e4m3fn [m, k] row-major (activations), ld_a bytes >= k, ld_a % 16 == 0;
 *   a_s: fp32 [k/128][ld_as], ld_as >= m (as written by fp8q_quant_act_g128);
 *   b:   e4m3fn [n, k] row-major (weights, nn.Linear [out, in]), ld_b >= k, ld_b % 16 == 0;
 *   b_s: fp32 [n/128][k/128] contiguous (as written by fp8q_quant_weight_blk128);
 *   y:   bf16 [m, n] row-major, ld_y elements >= n, ld_y % 8 == 0.
 *   n % 128 == 0, k % 128 == 0, k >= 128.  m == 0 is a no-op.  No bias.
 *   Each operand spans at most 2 GiB (else FP8Q_ERR_SHAPE): a (m * ld_a bytes), b
 *   (n * ld_b bytes) and a_s, addressed whole as 4 * ld_as * (k/128) bytes.
 * Accuracy: every element within half a bf16 ulp of the exact value plus 2e-3 of the
 * largest |y| (fp32 accumulation order differs from exact arithmetic).
 * ---------------------------------------------------------------------------- */
fp8q_status fp8q_gemm_w8a8_blkscaled(const void* a, int64_t ld_a, const float* a_s,
                                     int64_t ld_as, const void* b, int64_t ld_b,
                                     const float* b_s, void* y, int64_t ld_y, int64_t m,
                                     int64_t n, int64_t k, void* stream);

/* The block-scaled GEMM for power-of-two scales (as written by the *_ue8m0 quantizers):
 * same arguments, layouts, errors and accuracy bound as fp8q_gemm_w8a8_blkscaled.  The
 * matrix core applies the scales (E8M0 block-scaled MFMA) and accumulates across K
 * blocks directly.  Precondition (not checked): every a_s and b_s value is 2^e with
 * -127 <= e <= 127; other values are read as 2^(biased exponent field - 127). */
fp8q_status fp8q_gemm_w8a8_ue8m0(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                 const void* b, int64_t ld_b, const float* b_s, void* y,
                                 int64_t ld_y, int64_t m, int64_t n, int64_t k, void* stream);

/* ------------------------------------------------------------------------------
 * MoE grouped block-scaled W8A8 GEMM  [FP8-RL, "Method step details" step 1 (MoE
 * expert layers fc1, fc2); "Experimental results" (MoE gains)]
 *
 * Rows of `a` are sorted by expert: rows [offsets[g], offsets[g+1]) belong to expert g
 * and are multiplied by that expert's weight b[g] with scales b_s[g], exactly as in
 * fp8q_gemm_w8a8_blkscaled:
 *   a:   e4m3fn [total_m, k], ld_a bytes; a_s: fp32 [k/128][ld_as], ld_as >= total_m;
 *   b:   e4m3fn [G][n][k] contiguous; b_s: fp32 [G][n/128][k/128] contiguous;
 *   group_offsets: int32 [G+1] (device), read on the device only (no host sync);
 *   y:   bf16 [total_m, n], ld_y elements.
 * Empty groups are allowed.  num_groups >= 1; n, k multiples of 128; total_m == 0 is a
 * no-op.  Rows outside [offsets[0], offsets[G]) are not written.  As for the dense call,
 * total_m * ld_a, n * k (one expert) and 4 * ld_as * (k/128) bytes (the whole a_s) are
 * each at most 2 GiB.
 * ---------------------------------------------------------------------------- */
fp8q_status fp8q_grouped_gemm_w8a8(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                   const void* b, const float* b_s,
                                   const int32_t* group_offsets, int32_t num_groups,
                                   int64_t total_m, void* y, int64_t ld_y, int64_t n, int64_t k,
                                   void* stream);

/* fp8q_gemm_w8a8_bf16act: the few-token GEMM with the activation quantization fused into
 * its operand load [FP8-RL, "Method step details" step 1: activations quantized on every
 * forward].  x is bf16 [m][ld_x]; each 1x128 group of each row is quantized inside the GEMM
 * with the quantization rule above, exactly as fp8q_quant_act_g128 would, and y is what
 * fp8q_gemm_w8a8_blkscaled computes from those codes and scales: the result is bit-identical
 * to fp8q_quant_act_g128 followed by fp8q_gemm_w8a8_blkscaled.  The quantized activations
 * are not written anywhere.
 * 0 <= m <= 64 (decode and short prefill; for more tokens quantize once and call the GEMM:
 * every workgroup of this kernel quantizes its token rows again).  It saves time over the
 * two calls only for m <= 4 on one MI355X (m = 1, n = k = 4096: 5.9 against 7.6 us); from
 * m = 16 the two calls are faster (m = 16: 8.3 against 13.6 us), since the repeated
 * quantization grows with m while the two calls' extra launch does not.  n, k positive multiples
 * of 128; ld_x >= k with ld_x % 8 == 0; x and y 16-byte aligned; b, b_s, y and their
 * strides as for fp8q_gemm_w8a8_blkscaled.  m == 0 is a no-op. */
fp8q_status fp8q_gemm_w8a8_bf16act(const void* x, int64_t ld_x, const void* b, int64_t ld_b,
                                   const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                                   int64_t k, void* stream);

/* The same for power-of-two (UE8M0) scales: the token groups are quantized as
 * fp8q_quant_act_g128_ue8m0 would, and the result is bit-identical to that call followed
 * by fp8q_gemm_w8a8_ue8m0.  b_s precondition as fp8q_gemm_w8a8_ue8m0; other arguments,
 * limits and errors as fp8q_gemm_w8a8_bf16act. */
fp8q_status fp8q_gemm_w8a8_bf16act_ue8m0(const void* x, int64_t ld_x, const void* b, int64_t ld_b,
                                         const float* b_s, void* y, int64_t ld_y, int64_t m,
                                         int64_t n, int64_t k, void* stream);

/* fp8q_grouped_gemm_swiglu_quant: MoE fc1 with the SwiGLU activation and fc2's 1x128
 * input quantization fused into the GEMM's epilogue [R3, section 4: the grouped expert
 * GEMM over the recorded routing; Rounding, the SwiGLU fusion region: silu(gate) is
 * multiplied by up before any rounding; FP8-RL, "Method step details" step 1: fc2's
 * input is quantized per 1x128 group on every forward].
 * b is e4m3 [G][2*n_half][k]: per expert the gate rows 0..n_half-1, then the up rows;
 * b_s fp32 [G][2*n_half/128][k/128].  The results equal, bit for bit, the two calls
 *   fp8q_grouped_gemm_w8a8(a, ..., b, b_s, ..., y, ld_y = 2*n_half, n = 2*n_half, k)
 *   fp8q_swiglu_quant_g128(y, total_m, n_half, 2*n_half, q, ld_q, s, ld_s)
 * (the GEMM's outputs rounded to bf16 once, then SwiGLU and the quantization exactly as
 * fp8q_swiglu_quant_g128 defines them), without the bf16 buffer y: q receives e4m3 codes
 * [total_m][ld_q], n_half per row; s receives the scale of group g of row m at
 * s[g * ld_s + m].  The 256x256 tiles each take 128 gate and the matching 128 up rows.
 * Rows of a: with row_token NULL, a and a_s hold the total_m dispatched rows
 * (fp8q_moe_dispatch's aq and as; token_rows is ignored).  Otherwise a and a_s hold
 * token_rows token rows (fp8q_quant_act_g128's output, not copied), and dispatched row r
 * reads a[row_token[r]] and a_s[g][row_token[r]] (fp8q_moe_route's row_token): the
 * results are those of the dispatched-row call.  Precondition: 0 <= row_token[r] <
 * token_rows for r < total_m.
 * n_half and k positive multiples of 128, 2*n_half*k <= 2^31; ld_q >= n_half,
 * ld_s >= total_m, ld_as >= the rows of a; a, b, q 16-byte aligned with ld_a and ld_q
 * multiples of 16; the other arguments and preconditions as fp8q_grouped_gemm_w8a8 and
 * fp8q_swiglu_quant_g128 (the amax / 448 of every group fits binary32; debug mode cannot
 * check this one, which needs the GEMM's outputs).  total_m == 0 is a no-op. */
fp8q_status fp8q_grouped_gemm_swiglu_quant(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                           const int32_t* row_token, int64_t token_rows, const void* b,
                                           const float* b_s, const int32_t* group_offsets,
                                           int32_t num_groups, int64_t total_m, void* q, int64_t ld_q,
                                           float* s, int64_t ld_s, int64_t n_half, int64_t k,
                                           void* stream);

/* The same for power-of-two (UE8M0) scales: a_s and b_s as for
 * fp8q_grouped_gemm_w8a8_ue8m0 (precondition: every value is 2^e, -127 <= e <= 127), and
 * the epilogue quantizes as fp8q_swiglu_quant_g128_ue8m0.  The results equal, bit for bit,
 *   fp8q_grouped_gemm_w8a8_ue8m0(...) then fp8q_swiglu_quant_g128_ue8m0(...)
 * with the arguments of the fp32-scale composition above. */
fp8q_status fp8q_grouped_gemm_swiglu_quant_ue8m0(const void* a, int64_t ld_a, const float* a_s,
                                                 int64_t ld_as, const int32_t* row_token,
                                                 int64_t token_rows, const void* b, const float* b_s,
                                                 const int32_t* group_offsets, int32_t num_groups,
                                                 int64_t total_m, void* q, int64_t ld_q, float* s,
                                                 int64_t ld_s, int64_t n_half, int64_t k,
                                                 void* stream);

/* The grouped GEMM for power-of-two scales; arguments as fp8q_grouped_gemm_w8a8, scale
 * precondition as fp8q_gemm_w8a8_ue8m0. */
fp8q_status fp8q_grouped_gemm_w8a8_ue8m0(const void* a, int64_t ld_a, const float* a_s,
                                         int64_t ld_as, const void* b, const float* b_s,
                                         const int32_t* group_offsets, int32_t num_groups,
                                         int64_t total_m, void* y, int64_t ld_y, int64_t n,
                                         int64_t k, void* stream);

/* ------------------------------------------------------------------------------
 * FP8 KV cache quantize-on-write with per-step scale recalibration  [FP8-RL, "Method
 * step details" step 3; 1T-RL, 3.4]
 *
 * For each token t < num_tokens with slot = slot_mapping[t] >= 0 (a negative slot skips
 * the token), head h and dim d:
 *   k_cache[((slot / page_size) * page_size + slot % page_size) * H * D + h * D + d]
 *       = code of k[t * ld_k + h * D + d] / *k_scale,   and likewise for v.
 * Caches are e4m3fn [num_pages][page_size][H][D]; bytes of slots not written stay as
 * they were.  H = num_kv_heads >= 1, D = head_dim == 128.
 *   k, v: bf16 [num_tokens][ld_k] / [num_tokens][ld_v], ld >= H*D, ld % 8 == 0.
 *   slot_mapping: int64 [num_tokens] (device).
 *   k_scale, v_scale: one fp32 each (device), in/out.
 * flags & FP8Q_KV_RECALIBRATE: first set *k_scale = fl32(amax_K / fp8_range) and
 *   *v_scale = fl32(amax_V / fp8_range), amax over every element this call writes
 *   (1.0 when it is 0), then write with those scales (the first write of an RL step).
 * flags == 0: write with the stored *k_scale, *v_scale (later decode steps), which
 *   must be positive and finite; values beyond the E4M3 range saturate to +-448.
 * While a recalibrating call runs, *k_scale and *v_scale hold an intermediate value
 * (the amax with the sign bit set); the call's last kernel replaces it with the scale.
 * fp8_range > 0 and finite (448 maps amax onto the E4M3 maximum).
 * ---------------------------------------------------------------------------- */
#define FP8Q_KV_RECALIBRATE 1u

fp8q_status fp8q_kv_quant(const void* k, int64_t ld_k, const void* v, int64_t ld_v,
                          int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                          const int64_t* slot_mapping, void* k_cache, void* v_cache,
                          int32_t page_size, int64_t num_pages, float* k_scale, float* v_scale,
                          float fp8_range, uint32_t flags, void* stream);

/* ------------------------------------------------------------------------------
 * FP8 paged decode attention with per-step query-scale recalibration  [FP8-RL, "Method
 * step details" step 3 (Q/K/V scales recalibrated before every RL step's rollout) and
 * "Experimental results" (full FP8: linear layers, KV cache and attention); 1T-RL, 3.4]
 *
 * One decode query per sequence b and query head h; h reads KV head h / (H / Hkv).
 * The context of sequence b is its tokens t < seq_lens[b], token t in page
 * block_table[b * ld_bt + t / page_size], slot t % page_size, of caches laid out as
 * fp8q_kv_quant writes them (e4m3fn [num_pages][page_size][Hkv][128]).
 *   cq[d]  = E4M3 code of q[b][h][d] / *q_scale (the quantization rule above, saturating);
 *   s_t    = sm_scale * q_scale * k_scale * sum_d dec(cq[d]) * dec(ck[t][d]);
 *   out[d] = bf16( v_scale * sum_t softmax(s)_t * dec(cv[t][d]) ), softmax and sums in fp32.
 * q: bf16 [num_seqs][ld_q], the H query heads of a sequence contiguous (ld_q >= H*128,
 * ld_q % 8 == 0); out: bf16 [num_seqs][ld_out], same layout.  seq_lens: int32 [num_seqs];
 * a sequence with length <= 0 gets a zero output.  block_table: int32 [num_seqs][ld_bt].
 * q_scale, k_scale, v_scale: one fp32 each (device); k_scale and v_scale are the cache's
 * (fp8q_kv_quant's), positive and finite.
 * flags & FP8Q_ATTN_RECALIBRATE_Q: first set *q_scale = fl32(amax / fp8_range) over all
 *   num_seqs * H * 128 query values (1.0 if amax == 0), then attend with it (the first
 *   decode step of an RL step); flags == 0: use the stored *q_scale, which must be
 *   positive and finite (query values beyond its range saturate to +-448 codes).
 * head_dim == 128; 1 <= H / Hkv <= 16 with H a multiple of Hkv; page_size >= 1;
 * q, out and the caches 16-byte aligned.  Preconditions not checked: every page id is
 * below num_pages and every length at most ld_bt * page_size.
 * ---------------------------------------------------------------------------- */
#define FP8Q_ATTN_RECALIBRATE_Q 1u

fp8q_status fp8q_paged_decode_attention(const void* q, int64_t ld_q, const void* k_cache,
                                        const void* v_cache, const int32_t* block_table,
                                        int64_t ld_bt, const int32_t* seq_lens, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t page_size, int64_t num_pages, float* q_scale,
                                        const float* k_scale, const float* v_scale, float sm_scale,
                                        float fp8_range, uint32_t flags, void* out, int64_t ld_out,
                                        void* stream);

/* ------------------------------------------------------------------------------
 * MoE layer around the grouped GEMM  [R3, "Rollout Routing Replay" and the cost
 * analysis: each token's top-k expert indices are recorded as int16 and tokens are
 * dispatched to exactly those experts; Rounding, SwiGLU fusion region; FP8-RL step 1]
 *
 * fp8q_moe_dispatch: gathers quantized token rows (and their 1x128 scales) into
 * expert-sorted rows for fp8q_grouped_gemm_w8a8.
 *   topk_ids: int16 [num_tokens][topk] (device, contiguous, 16-byte aligned).  Entry
 *     f = t*topk + j is valid when 0 <= topk_ids[f] < num_experts; invalid entries are
 *     dropped.  Valid entries are ordered by expert id and, within an expert, by f.
 *   xq: e4m3fn [num_tokens][ld_xq], xs: fp32 [k/128][ld_xs] (the layout of
 *     fp8q_quant_act_g128's output), ld_xq >= k, ld_xs >= num_tokens.
 *   aq: e4m3fn [R][ld_aq], as: fp32 [k/128][ld_as], R = number of valid entries
 *     <= num_tokens*topk, ld_as >= num_tokens*topk: row r of aq is token f/topk's codes
 *     for the r-th entry in that order, as[g][r] its scale of group g.
 *   offsets: int32 [num_experts + 1] (out): rows of expert e are [offsets[e],
 *     offsets[e+1]); offsets[0] = 0, offsets[num_experts] = R.
 *   row_of: int32 [num_tokens*topk] (out): the row of entry f, -1 if dropped.
 * k a positive multiple of 128; topk >= 1; 1 <= num_experts <= 32767;
 * num_tokens * topk < 2^31.  xq/aq 16-byte aligned with ld_xq, ld_aq multiples of 16.
 * num_tokens == 0 writes offsets (all 0) only.
 * ---------------------------------------------------------------------------- */
fp8q_status fp8q_moe_dispatch(const void* xq, int64_t ld_xq, const float* xs, int64_t ld_xs,
                              const int16_t* topk_ids, int64_t num_tokens, int32_t topk,
                              int32_t num_experts, int64_t k, void* aq, int64_t ld_aq, float* as,
                              int64_t ld_as, int32_t* offsets, int32_t* row_of, void* stream);

/* fp8q_moe_route: the routing step of fp8q_moe_dispatch without the copies, for a fc1
 * that reads each dispatched row straight from the token matrix
 * (fp8q_grouped_gemm_swiglu_quant with row_token).  offsets and row_of are exactly
 * those fp8q_moe_dispatch writes; row_token: int32 [num_tokens*topk] (out), its first
 * R entries set: row_token[r] = the token of row r (row_token[row_of[f]] = f / topk).
 * Arguments and limits as fp8q_moe_dispatch; row_token 4-byte aligned. */
fp8q_status fp8q_moe_route(const int16_t* topk_ids, int64_t num_tokens, int32_t topk, int32_t num_experts,
                           int32_t* offsets, int32_t* row_of, int32_t* row_token, void* stream);

/* fp8q_swiglu_quant_g128: h = [gate | up], bf16 [m][ld_h] with gate in columns [0, n)
 * and up in [n, 2n) (fc1's output); a = silu(gate) * up = gate / (1 + exp(-gate)) * up,
 * formed in fp64 and never rounded before the quantization; then the quantization rule
 * above per row and 128-column group: amax = max |a|, scale = fl32(fl64(amax / 448))
 * (1.0 if amax == 0), code = the E4M3FN value nearest the fp64 quotient a / scale.
 * Output layout as fp8q_quant_act_g128: q e4m3fn [m][ld_q], s[g * ld_s + row].
 * n a multiple of 128; ld_h >= 2n, ld_h % 8 == 0; ld_q >= n, ld_q % 16 == 0; ld_s >= m;
 * h, q 16-byte aligned.  Precondition: amax / 448 fits binary32. */
fp8q_status fp8q_swiglu_quant_g128(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q,
                                   int64_t ld_q, float* s, int64_t ld_s, void* stream);

/* The same with power-of-two (UE8M0) scales [FP8-RL, "Experimental results", scale-format
 * ablation], so that fc2 can run as fp8q_grouped_gemm_w8a8_ue8m0: scale = the smallest
 * 2^e with 448 * 2^e >= amax (exact comparison with the fp64 amax), e limited to
 * [-127, 127], 1.0 if amax == 0; code = the E4M3FN value nearest the exact quotient
 * a / scale (saturating).  Arguments, layouts and errors as fp8q_swiglu_quant_g128,
 * without the binary32 precondition. */
fp8q_status fp8q_swiglu_quant_g128_ue8m0(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q,
                                         int64_t ld_q, float* s, int64_t ld_s, void* stream);

/* fp8q_moe_combine: out[t][c] = bf16( sum_{j < topk, row_of[t*topk+j] >= 0}
 *   weights[t*topk+j] * y[row_of[t*topk+j]][c] ), the sum in fp32 in the order of j
 * (one fused multiply-add per term), rounded to bf16 (nearest even) once.
 *   y: bf16 [rows][ld_y] (fc2's output in dispatch order); row_of: int32
 *   [num_tokens*topk] (fp8q_moe_dispatch's); weights: fp32 [num_tokens*topk];
 *   out: bf16 [num_tokens][ld_out].
 * hidden a positive multiple of 8; ld_y, ld_out >= hidden and multiples of 8; y, out
 * 16-byte aligned.  Precondition: every row_of entry is -1 or below the rows of y. */
fp8q_status fp8q_moe_combine(const void* y, int64_t ld_y, const int32_t* row_of, const float* weights,
                             int64_t num_tokens, int32_t topk, int64_t hidden, void* out,
                             int64_t ld_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */

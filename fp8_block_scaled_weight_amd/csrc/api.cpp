// C ABI of libfp8q: host-side argument validation and kernel dispatch.
// The contract of every entry point is documented in include/fp8q.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fp8q.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

fp8q_status fail(fp8q_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

fp8q_status ok() {
  g_err[0] = '\0';
  return FP8Q_OK;
}

// The GEMM kernels address each operand with 32-bit byte offsets.
constexpr int64_t kMaxOperandBytes = (int64_t)1 << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];

fp8q_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(FP8Q_ERR_UNSUPPORTED, "no HIP device available");
  }
  if (dev >= kMaxDevices) return fail(FP8Q_ERR_UNSUPPORTED, "device index %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(FP8Q_ERR_UNSUPPORTED, "cannot query device %d", dev);
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(FP8Q_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return FP8Q_OK;
}

fp8q_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP8Q_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* fp8q_status_string(fp8q_status s) {
  switch (s) {
    case FP8Q_OK: return "FP8Q_OK";
    case FP8Q_ERR_NULL: return "FP8Q_ERR_NULL";
    case FP8Q_ERR_SHAPE: return "FP8Q_ERR_SHAPE";
    case FP8Q_ERR_STRIDE: return "FP8Q_ERR_STRIDE";
    case FP8Q_ERR_ALIGN: return "FP8Q_ERR_ALIGN";
    case FP8Q_ERR_LAUNCH: return "FP8Q_ERR_LAUNCH";
    case FP8Q_ERR_UNSUPPORTED: return "FP8Q_ERR_UNSUPPORTED";
  }
  return "FP8Q_(unknown status)";
}

const char* fp8q_last_error(void) { return g_err; }

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

static fp8q_status quant_weight(const fp8q_weight_desc* descs, int32_t count, void* stream, bool pow2) {
  if (count < 1) return fail(FP8Q_ERR_SHAPE, "count must be >= 1 (got %d)", count);
  if (!descs) return fail(FP8Q_ERR_NULL, "descs is NULL");
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    const fp8q_weight_desc& d = descs[i];
    if (d.n < 0 || d.k < 0) return fail(FP8Q_ERR_SHAPE, "desc %d: negative shape", i);
    if (d.n % 128 || d.k % 128)
      return fail(FP8Q_ERR_SHAPE, "desc %d: n=%lld and k=%lld must be multiples of 128", i, (long long)d.n,
                  (long long)d.k);
    if (d.n == 0 || d.k == 0) continue;
    if (!d.w || !d.q || !d.s) return fail(FP8Q_ERR_NULL, "desc %d: NULL pointer", i);
    if (d.ld_w < d.k || d.ld_q < d.k) return fail(FP8Q_ERR_STRIDE, "desc %d: ld_w/ld_q smaller than k", i);
    if (!aligned16(d.w) || !aligned16(d.q) || d.ld_w % 8 || d.ld_q % 16 || !aligned4(d.s))
      return fail(FP8Q_ERR_ALIGN, "desc %d: w/q must be 16-byte aligned with ld_w %% 8 == 0, ld_q %% 16 == 0", i);
    total += (d.n / 128) * (d.k / 128);
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  if (total == 0) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  fp8q::WeightChunk chunk;
  chunk.count = 0;
  int64_t blocks = 0;
  for (int32_t i = 0; i < count; ++i) {
    const fp8q_weight_desc& d = descs[i];
    if (d.n == 0 || d.k == 0) continue;
    const int64_t nblk = (d.n / 128) * (d.k / 128);
    if (chunk.count == fp8q::kWeightChunk || blocks + nblk > (int64_t)0x7fffffff) {
      st = launched(fp8q::launch_quant_weight_chunk(chunk, blocks, pow2, s), "quant_weight_blk128");
      if (st != FP8Q_OK) return st;
      chunk.count = 0;
      blocks = 0;
    }
    fp8q::WeightDescDev& e = chunk.d[chunk.count++];
    e.w = d.w;
    e.q = d.q;
    e.s = d.s;
    e.ld_w = d.ld_w;
    e.ld_q = d.ld_q;
    e.first_block = (int32_t)blocks;
    e.kblocks = (int32_t)(d.k / 128);
    blocks += nblk;
  }
  return launched(fp8q::launch_quant_weight_chunk(chunk, blocks, pow2, s), "quant_weight_blk128");
}

fp8q_status fp8q_quant_weight_blk128(const fp8q_weight_desc* descs, int32_t count, void* stream) {
  return quant_weight(descs, count, stream, false);
}

fp8q_status fp8q_quant_weight_blk128_ue8m0(const fp8q_weight_desc* descs, int32_t count, void* stream) {
  return quant_weight(descs, count, stream, true);
}

static fp8q_status quant_act(const void* x, int64_t m, int64_t k, int64_t ld_x, void* q, int64_t ld_q, float* s,
                             int64_t ld_s, void* stream, bool pow2) {
  if (m < 0 || k < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (k % 128) return fail(FP8Q_ERR_SHAPE, "k=%lld must be a multiple of 128", (long long)k);
  if (m == 0 || k == 0) {
    fp8q_status st = check_device();
    return st == FP8Q_OK ? ok() : st;
  }
  if (!x || !q || !s) return fail(FP8Q_ERR_NULL, "NULL pointer");
  if (ld_x < k || ld_q < k || ld_s < m) return fail(FP8Q_ERR_STRIDE, "ld_x/ld_q < k or ld_s < m");
  if (!aligned16(x) || !aligned16(q) || ld_x % 8 || ld_q % 16 || !aligned4(s))
    return fail(FP8Q_ERR_ALIGN, "x/q must be 16-byte aligned with ld_x %% 8 == 0 and ld_q %% 16 == 0");
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_quant_act(x, m, k, ld_x, q, ld_q, s, ld_s, pow2, reinterpret_cast<hipStream_t>(stream)),
                  "quant_act_g128");
}

fp8q_status fp8q_quant_act_g128(const void* x, int64_t m, int64_t k, int64_t ld_x, void* q, int64_t ld_q,
                                float* s, int64_t ld_s, void* stream) {
  return quant_act(x, m, k, ld_x, q, ld_q, s, ld_s, stream, false);
}

fp8q_status fp8q_quant_act_g128_ue8m0(const void* x, int64_t m, int64_t k, int64_t ld_x, void* q, int64_t ld_q,
                                      float* s, int64_t ld_s, void* stream) {
  return quant_act(x, m, k, ld_x, q, ld_q, s, ld_s, stream, true);
}

static fp8q_status check_gemm_common(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                     const void* y, int64_t ld_y, int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (n % 128 || k % 128 || n == 0 || k == 0)
    return fail(FP8Q_ERR_SHAPE, "n=%lld and k=%lld must be positive multiples of 128", (long long)n,
                (long long)k);
  if (m == 0) return FP8Q_OK;
  if (!a || !a_s || !y) return fail(FP8Q_ERR_NULL, "NULL pointer");
  if (ld_a < k || ld_as < m || ld_y < n) return fail(FP8Q_ERR_STRIDE, "ld_a < k, ld_as < m or ld_y < n");
  if (!aligned16(a) || !aligned16(y) || ld_a % 16 || ld_y % 8 || !aligned4(a_s))
    return fail(FP8Q_ERR_ALIGN, "a/y must be 16-byte aligned with ld_a %% 16 == 0 and ld_y %% 8 == 0");
  if (m * ld_a > kMaxOperandBytes || ld_as * 4 > kMaxOperandBytes)
    return fail(FP8Q_ERR_SHAPE, "an operand spans more than 2 GiB");
  return FP8Q_OK;
}

static fp8q_status gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b, int64_t ld_b,
                        const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n, int64_t k, void* stream,
                        bool pow2) {
  fp8q_status st = check_gemm_common(a, ld_a, a_s, ld_as, y, ld_y, m, n, k);
  if (st != FP8Q_OK) return st;
  if (m > 0) {
    if (!b || !b_s) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (ld_b < k) return fail(FP8Q_ERR_STRIDE, "ld_b < k");
    if (!aligned16(b) || ld_b % 16 || !aligned4(b_s))
      return fail(FP8Q_ERR_ALIGN, "b must be 16-byte aligned with ld_b %% 16 == 0");
    if (n * ld_b > kMaxOperandBytes) return fail(FP8Q_ERR_SHAPE, "b spans more than 2 GiB");
  }
  st = check_device();
  if (st != FP8Q_OK) return st;
  if (m == 0) return ok();
  return launched(fp8q::launch_gemm(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, pow2,
                                    reinterpret_cast<hipStream_t>(stream)),
                  "gemm_w8a8_blkscaled");
}

fp8q_status fp8q_gemm_w8a8_blkscaled(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                     const void* b, int64_t ld_b, const float* b_s, void* y, int64_t ld_y,
                                     int64_t m, int64_t n, int64_t k, void* stream) {
  return gemm(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream, false);
}

fp8q_status fp8q_gemm_w8a8_ue8m0(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                 int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                                 int64_t k, void* stream) {
  return gemm(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream, true);
}

fp8q_status fp8q_gemm_w8a8_bf16act(const void* x, int64_t ld_x, const void* b, int64_t ld_b, const float* b_s,
                                   void* y, int64_t ld_y, int64_t m, int64_t n, int64_t k, void* stream) {
  if (m < 0 || n < 0 || k < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (m > 64) return fail(FP8Q_ERR_SHAPE, "m=%lld: the fused activation quantization takes at most 64 tokens",
                          (long long)m);
  if (n % 128 || k % 128 || n == 0 || k == 0)
    return fail(FP8Q_ERR_SHAPE, "n=%lld and k=%lld must be positive multiples of 128", (long long)n, (long long)k);
  if (m > 0) {
    if (!x || !b || !b_s || !y) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (ld_x < k || ld_b < k || ld_y < n) return fail(FP8Q_ERR_STRIDE, "ld_x < k, ld_b < k or ld_y < n");
    if (!aligned16(x) || !aligned16(b) || !aligned16(y) || ld_x % 8 || ld_b % 16 || ld_y % 8 || !aligned4(b_s))
      return fail(FP8Q_ERR_ALIGN, "x/b/y must be 16-byte aligned with ld_x %% 8, ld_b %% 16, ld_y %% 8 == 0");
    if (n * ld_b > kMaxOperandBytes) return fail(FP8Q_ERR_SHAPE, "b spans more than 2 GiB");
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  if (m == 0) return ok();
  return launched(fp8q::launch_gemm_bf16act(x, ld_x, b, ld_b, b_s, y, ld_y, m, n, k,
                                            reinterpret_cast<hipStream_t>(stream)),
                  "gemm_w8a8_bf16act");
}

static fp8q_status grouped_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                const float* b_s, const int32_t* group_offsets, int32_t num_groups, int64_t total_m,
                                void* y, int64_t ld_y, int64_t n, int64_t k, void* stream, bool pow2) {
  if (num_groups < 1) return fail(FP8Q_ERR_SHAPE, "num_groups must be >= 1 (got %d)", num_groups);
  fp8q_status st = check_gemm_common(a, ld_a, a_s, ld_as, y, ld_y, total_m, n, k);
  if (st != FP8Q_OK) return st;
  if (total_m > 0) {
    if (!b || !b_s || !group_offsets) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (!aligned16(b) || !aligned4(b_s) || !aligned4(group_offsets))
      return fail(FP8Q_ERR_ALIGN, "b must be 16-byte aligned");
    if (n * k > kMaxOperandBytes) return fail(FP8Q_ERR_SHAPE, "one expert's weight spans more than 2 GiB");
  }
  st = check_device();
  if (st != FP8Q_OK) return st;
  if (total_m == 0) return ok();
  return launched(fp8q::launch_grouped_gemm(a, ld_a, a_s, ld_as, b, b_s, group_offsets, num_groups, total_m, y,
                                            ld_y, n, k, pow2, reinterpret_cast<hipStream_t>(stream)),
                  "grouped_gemm_w8a8");
}

fp8q_status fp8q_grouped_gemm_w8a8(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                   const float* b_s, const int32_t* group_offsets, int32_t num_groups,
                                   int64_t total_m, void* y, int64_t ld_y, int64_t n, int64_t k, void* stream) {
  return grouped_gemm(a, ld_a, a_s, ld_as, b, b_s, group_offsets, num_groups, total_m, y, ld_y, n, k, stream, false);
}

fp8q_status fp8q_grouped_gemm_w8a8_ue8m0(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                         const void* b, const float* b_s, const int32_t* group_offsets,
                                         int32_t num_groups, int64_t total_m, void* y, int64_t ld_y, int64_t n,
                                         int64_t k, void* stream) {
  return grouped_gemm(a, ld_a, a_s, ld_as, b, b_s, group_offsets, num_groups, total_m, y, ld_y, n, k, stream, true);
}

fp8q_status fp8q_kv_quant(const void* k, int64_t ld_k, const void* v, int64_t ld_v, int64_t num_tokens,
                          int32_t num_kv_heads, int32_t head_dim, const int64_t* slot_mapping, void* k_cache,
                          void* v_cache, int32_t page_size, int64_t num_pages, float* k_scale, float* v_scale,
                          float fp8_range, uint32_t flags, void* stream) {
  if (num_tokens < 0 || num_pages < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (num_kv_heads < 1) return fail(FP8Q_ERR_SHAPE, "num_kv_heads must be >= 1");
  if (head_dim != 128) return fail(FP8Q_ERR_SHAPE, "head_dim must be 128 (got %d)", head_dim);
  if (page_size < 1) return fail(FP8Q_ERR_SHAPE, "page_size must be >= 1");
  if (!(fp8_range > 0.0f) || fp8_range > 3.4e38f) return fail(FP8Q_ERR_SHAPE, "fp8_range must be positive and finite");
  if (flags & ~FP8Q_KV_RECALIBRATE) return fail(FP8Q_ERR_SHAPE, "unknown flag bits 0x%x", flags);
  const int64_t row = (int64_t)num_kv_heads * head_dim;
  if (!k_scale || !v_scale) return fail(FP8Q_ERR_NULL, "k_scale/v_scale is NULL");
  if (num_tokens > 0) {
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (ld_k < row || ld_v < row) return fail(FP8Q_ERR_STRIDE, "ld_k/ld_v smaller than heads*head_dim");
    if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache) || ld_k % 8 || ld_v % 8 ||
        !aligned4(k_scale) || !aligned4(v_scale) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
      return fail(FP8Q_ERR_ALIGN, "k/v/caches must be 16-byte aligned with ld_k %% 8 == 0 and ld_v %% 8 == 0");
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  if (num_tokens == 0 && !(flags & FP8Q_KV_RECALIBRATE)) return ok();
  return launched(fp8q::launch_kv_quant(k, ld_k, v, ld_v, num_tokens, num_kv_heads, slot_mapping, k_cache, v_cache,
                                        k_scale, v_scale, fp8_range, (flags & FP8Q_KV_RECALIBRATE) != 0,
                                        reinterpret_cast<hipStream_t>(stream)),
                  "kv_quant");
}

fp8q_status fp8q_moe_dispatch(const void* xq, int64_t ld_xq, const float* xs, int64_t ld_xs, const int16_t* topk_ids,
                              int64_t num_tokens, int32_t topk, int32_t num_experts, int64_t k, void* aq,
                              int64_t ld_aq, float* as, int64_t ld_as, int32_t* offsets, int32_t* row_of,
                              void* stream) {
  if (num_tokens < 0 || k < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (topk < 1) return fail(FP8Q_ERR_SHAPE, "topk must be >= 1 (got %d)", topk);
  if (num_experts < 1 || num_experts > 32767)
    return fail(FP8Q_ERR_SHAPE, "num_experts must be in [1, 32767] (got %d)", num_experts);
  if (k == 0 || k % 128) return fail(FP8Q_ERR_SHAPE, "k=%lld must be a positive multiple of 128", (long long)k);
  const int64_t n = num_tokens * (int64_t)topk;
  if (n > 0x7fffffffLL) return fail(FP8Q_ERR_SHAPE, "num_tokens * topk must be below 2^31");
  if (!offsets) return fail(FP8Q_ERR_NULL, "offsets is NULL");
  if (!aligned4(offsets)) return fail(FP8Q_ERR_ALIGN, "offsets must be 4-byte aligned");
  if (n > 0) {
    if (!xq || !xs || !topk_ids || !aq || !as || !row_of) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (ld_xq < k || ld_aq < k || ld_xs < num_tokens || ld_as < n)
      return fail(FP8Q_ERR_STRIDE, "ld_xq/ld_aq < k, ld_xs < num_tokens or ld_as < num_tokens*topk");
    if (!aligned16(xq) || !aligned16(aq) || ld_xq % 16 || ld_aq % 16 || !aligned16(topk_ids) || !aligned4(xs) ||
        !aligned4(as) || !aligned4(row_of))
      return fail(FP8Q_ERR_ALIGN, "xq/aq/topk_ids must be 16-byte aligned with ld_xq, ld_aq multiples of 16");
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_moe_dispatch(xq, ld_xq, xs, ld_xs, topk_ids, num_tokens, topk, num_experts, k, aq,
                                            ld_aq, as, ld_as, offsets, row_of, reinterpret_cast<hipStream_t>(stream)),
                  "moe_dispatch");
}

fp8q_status fp8q_swiglu_quant_g128(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q, int64_t ld_q,
                                   float* s, int64_t ld_s, void* stream) {
  if (m < 0 || n < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (n % 128) return fail(FP8Q_ERR_SHAPE, "n=%lld must be a multiple of 128", (long long)n);
  if (m == 0 || n == 0) {
    fp8q_status st = check_device();
    return st == FP8Q_OK ? ok() : st;
  }
  if (!h || !q || !s) return fail(FP8Q_ERR_NULL, "NULL pointer");
  if (ld_h < 2 * n || ld_q < n || ld_s < m) return fail(FP8Q_ERR_STRIDE, "ld_h < 2n, ld_q < n or ld_s < m");
  if (!aligned16(h) || !aligned16(q) || ld_h % 8 || ld_q % 16 || !aligned4(s))
    return fail(FP8Q_ERR_ALIGN, "h/q must be 16-byte aligned with ld_h %% 8 == 0 and ld_q %% 16 == 0");
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  return launched(fp8q::launch_swiglu_quant(h, m, n, ld_h, q, ld_q, s, ld_s, reinterpret_cast<hipStream_t>(stream)),
                  "swiglu_quant_g128");
}

fp8q_status fp8q_moe_combine(const void* y, int64_t ld_y, const int32_t* row_of, const float* weights,
                             int64_t num_tokens, int32_t topk, int64_t hidden, void* out, int64_t ld_out,
                             void* stream) {
  if (num_tokens < 0 || hidden < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (topk < 1) return fail(FP8Q_ERR_SHAPE, "topk must be >= 1 (got %d)", topk);
  if (hidden == 0 || hidden % 8)
    return fail(FP8Q_ERR_SHAPE, "hidden=%lld must be a positive multiple of 8", (long long)hidden);
  if (num_tokens > 0) {
    if (!y || !row_of || !weights || !out) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (ld_y < hidden || ld_out < hidden) return fail(FP8Q_ERR_STRIDE, "ld_y/ld_out < hidden");
    if (!aligned16(y) || !aligned16(out) || ld_y % 8 || ld_out % 8 || !aligned4(row_of) || !aligned4(weights))
      return fail(FP8Q_ERR_ALIGN, "y/out must be 16-byte aligned with ld_y, ld_out multiples of 8");
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  if (num_tokens == 0) return ok();
  return launched(fp8q::launch_moe_combine(y, ld_y, row_of, weights, num_tokens, topk, hidden, out, ld_out,
                                           reinterpret_cast<hipStream_t>(stream)),
                  "moe_combine");
}

fp8q_status fp8q_paged_decode_attention(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_table, int64_t ld_bt, const int32_t* seq_lens,
                                        int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t page_size, int64_t num_pages, float* q_scale,
                                        const float* k_scale, const float* v_scale, float sm_scale,
                                        float fp8_range, uint32_t flags, void* out, int64_t ld_out, void* stream) {
  if (num_seqs < 0 || num_pages < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (num_q_heads < 1 || num_kv_heads < 1 || num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > 16)
    return fail(FP8Q_ERR_SHAPE, "num_q_heads must be a multiple of num_kv_heads, at most 16 times it");
  if (head_dim != 128) return fail(FP8Q_ERR_SHAPE, "head_dim must be 128 (got %d)", head_dim);
  if (page_size < 1) return fail(FP8Q_ERR_SHAPE, "page_size must be >= 1");
  if (flags & ~FP8Q_ATTN_RECALIBRATE_Q) return fail(FP8Q_ERR_SHAPE, "unknown flag bits 0x%x", flags);
  if (!(fp8_range > 0.0f) || fp8_range > 3.4e38f) return fail(FP8Q_ERR_SHAPE, "fp8_range must be positive and finite");
  if (!(sm_scale == sm_scale) || sm_scale > 3.4e38f || sm_scale < -3.4e38f)
    return fail(FP8Q_ERR_SHAPE, "sm_scale must be finite");
  if (!q_scale || !k_scale || !v_scale) return fail(FP8Q_ERR_NULL, "q_scale/k_scale/v_scale is NULL");
  const int64_t row = (int64_t)num_q_heads * 128;
  if (num_seqs > 0) {
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (ld_q < row || ld_out < row || ld_bt < 1) return fail(FP8Q_ERR_STRIDE, "ld_q/ld_out < heads*128 or ld_bt < 1");
    if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache) || ld_q % 8 || ld_out % 8 ||
        !aligned4(block_table) || !aligned4(seq_lens) || !aligned4(q_scale) || !aligned4(k_scale) ||
        !aligned4(v_scale))
      return fail(FP8Q_ERR_ALIGN, "q/out/caches must be 16-byte aligned with ld_q, ld_out multiples of 8");
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  if (num_seqs == 0 && !(flags & FP8Q_ATTN_RECALIBRATE_Q)) return ok();
  return launched(fp8q::launch_decode_attention(q, ld_q, k_cache, v_cache, block_table, ld_bt, seq_lens, num_seqs,
                                                num_q_heads, num_kv_heads, page_size, q_scale, k_scale, v_scale,
                                                sm_scale, fp8_range, (flags & FP8Q_ATTN_RECALIBRATE_Q) != 0, out,
                                                ld_out, reinterpret_cast<hipStream_t>(stream)),
                  "paged_decode_attention");
}

}  // extern "C"

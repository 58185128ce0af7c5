// C ABI of libfp8q: host-side argument validation and kernel dispatch.
// The contract of every entry point is documented in include/fp8q.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <vector>

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

// ---------------------------------------------------------------- debug mode (FP8Q_DEBUG=1)
// Checks of the preconditions the kernels trust, before anything is enqueued; device data
// is read after synchronizing the call's stream.  After the launch the stream is
// synchronized again, so a device fault is reported by the call that caused it.

bool debug_on() {
  const char* e = std::getenv("FP8Q_DEBUG");
  return e && e[0] == '1' && e[1] == '\0';
}

// [lo, hi) byte extent of `rows` rows of `row_bytes` bytes, `pitch` bytes apart
struct Extent {
  uintptr_t lo = 0, hi = 0;
  const char* name = "";
};
Extent extent(const void* p, int64_t rows, int64_t row_bytes, int64_t pitch, const char* name) {
  Extent e;
  e.name = name;
  if (p && rows > 0 && row_bytes > 0) {
    e.lo = reinterpret_cast<uintptr_t>(p);
    e.hi = e.lo + static_cast<uintptr_t>((rows - 1) * pitch + row_bytes);
  }
  return e;
}
bool overlap(const Extent& a, const Extent& b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

fp8q_status check_disjoint(const std::vector<Extent>& outs, const std::vector<Extent>& ins) {
  for (size_t o = 0; o < outs.size(); ++o) {
    for (const Extent& i : ins)
      if (overlap(outs[o], i))
        return fail(FP8Q_ERR_PRECONDITION, "output %s overlaps input %s", outs[o].name, i.name);
    for (size_t o2 = o + 1; o2 < outs.size(); ++o2)
      if (overlap(outs[o], outs[o2]))
        return fail(FP8Q_ERR_PRECONDITION, "output %s overlaps output %s", outs[o].name, outs[o2].name);
  }
  return FP8Q_OK;
}

// settle the stream before reading device data; a capturing stream cannot be read
fp8q_status debug_sync(void* stream) {
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return fail(FP8Q_ERR_LAUNCH, "FP8Q_DEBUG: cannot query the stream");
  }
  if (cs != hipStreamCaptureStatusNone)
    return fail(FP8Q_ERR_UNSUPPORTED, "FP8Q_DEBUG=1 reads device data and cannot run on a capturing stream");
  const hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FP8Q_ERR_LAUNCH, "FP8Q_DEBUG: earlier work on the stream failed: %s", hipGetErrorString(e));
  }
  return FP8Q_OK;
}

// rows x cols elements of T, `ld` elements apart, copied to the host
template <class T>
fp8q_status fetch(std::vector<T>& out, const void* p, int64_t rows, int64_t cols, int64_t ld) {
  out.assign(static_cast<size_t>(rows > 0 && cols > 0 ? rows * cols : 0), T{});
  if (out.empty()) return FP8Q_OK;
  const hipError_t e = hipMemcpy2D(out.data(), cols * sizeof(T), p, ld * sizeof(T), cols * sizeof(T), rows,
                                   hipMemcpyDeviceToHost);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FP8Q_ERR_LAUNCH, "FP8Q_DEBUG: reading device data failed: %s", hipGetErrorString(e));
  }
  return FP8Q_OK;
}

fp8q_status finite_bf16(const void* p, int64_t rows, int64_t cols, int64_t ld, const char* name) {
  std::vector<uint16_t> v;
  fp8q_status st = fetch(v, p, rows, cols, ld);
  for (size_t i = 0; st == FP8Q_OK && i < v.size(); ++i)
    if ((v[i] & 0x7f80u) == 0x7f80u)
      return fail(FP8Q_ERR_PRECONDITION, "%s[%lld][%lld] is not finite (bf16 0x%04x)", name,
                  (long long)(i / cols), (long long)(i % cols), v[i]);
  return st;
}

// finite fp32 values; pow2: 2^e with -127 <= e <= 127 (normal, or the one subnormal
// 2^-127, whose E8M0 code is 0: smaller subnormals have no E8M0 code)
fp8q_status check_f32(const void* p, int64_t rows, int64_t cols, int64_t ld, const char* name, bool pow2,
                      bool positive) {
  std::vector<float> v;
  fp8q_status st = fetch(v, p, rows, cols, ld);
  for (size_t i = 0; st == FP8Q_OK && i < v.size(); ++i) {
    const float x = v[i];
    uint32_t b;
    std::memcpy(&b, &x, 4);
    const uint32_t man = b & 0x7fffffu, ex = (b >> 23) & 0xffu;
    const bool bad = !std::isfinite(x) || (positive && !(x > 0.0f)) ||
                     (pow2 && (!(x > 0.0f) || (ex != 0 ? man != 0 : man != 0x400000u)));
    if (bad)
      return fail(FP8Q_ERR_PRECONDITION, "%s[%lld][%lld] = %g is not %s", name, (long long)(i / cols),
                  (long long)(i % cols), (double)x,
                  pow2 ? "a positive power of two 2^e, -127 <= e <= 127" : (positive ? "positive and finite" : "finite"));
  }
  return st;
}

fp8q_status no_nan_codes(const void* p, int64_t rows, int64_t cols, int64_t ld, const char* name) {
  std::vector<uint8_t> v;
  fp8q_status st = fetch(v, p, rows, cols, ld);
  for (size_t i = 0; st == FP8Q_OK && i < v.size(); ++i)
    if ((v[i] & 0x7fu) == 0x7fu)
      return fail(FP8Q_ERR_PRECONDITION, "%s[%lld][%lld] is an E4M3 NaN code (0x%02x)", name,
                  (long long)(i / cols), (long long)(i % cols), v[i]);
  return st;
}

// after the launch: report a device fault of this call
fp8q_status finish(fp8q_status st, void* stream, const char* what) {
  if (st != FP8Q_OK || !debug_on()) return st;
  const hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(FP8Q_ERR_LAUNCH, "%s: device error: %s", what, hipGetErrorString(e));
  }
  return st;
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
    case FP8Q_ERR_PRECONDITION: return "FP8Q_ERR_PRECONDITION";
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
  if (debug_on()) {
    std::vector<Extent> outs, ins;
    for (int32_t i = 0; i < count; ++i) {
      const fp8q_weight_desc& d = descs[i];
      if (d.n == 0 || d.k == 0) continue;
      outs.push_back(extent(d.q, d.n, d.k, d.ld_q, "q"));
      outs.push_back(extent(d.s, 1, (d.n / 128) * (d.k / 128) * 4, 0, "s"));
      ins.push_back(extent(d.w, d.n, 2 * d.k, 2 * d.ld_w, "w"));
    }
    st = check_disjoint(outs, ins);
    if (st == FP8Q_OK) st = debug_sync(stream);
    for (int32_t i = 0; st == FP8Q_OK && i < count; ++i)
      if (descs[i].n > 0 && descs[i].k > 0) st = finite_bf16(descs[i].w, descs[i].n, descs[i].k, descs[i].ld_w, "w");
    if (st != FP8Q_OK) return st;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  fp8q::WeightChunk chunk;
  chunk.count = 0;
  int64_t blocks = 0, quads = 0;
  for (int32_t i = 0; i < count; ++i) {
    const fp8q_weight_desc& d = descs[i];
    if (d.n == 0 || d.k == 0) continue;
    const int64_t nblk = (d.n / 128) * (d.k / 128);
    const int64_t nquad = (d.n / 128) * ((d.k / 128 + 3) / 4);
    if (chunk.count == fp8q::kWeightChunk || blocks + nblk > (int64_t)0x7fffffff) {
      st = launched(fp8q::launch_quant_weight_chunk(chunk, blocks, quads, pow2, s), "quant_weight_blk128");
      if (st != FP8Q_OK) return st;
      chunk.count = 0;
      blocks = 0;
      quads = 0;
    }
    fp8q::WeightDescDev& e = chunk.d[chunk.count++];
    e.w = d.w;
    e.q = d.q;
    e.s = d.s;
    e.ld_w = d.ld_w;
    e.ld_q = d.ld_q;
    e.first_block = (int32_t)blocks;
    e.kblocks = (int32_t)(d.k / 128);
    e.first_quad = (int32_t)quads;
    e.kquads = (int32_t)((d.k / 128 + 3) / 4);
    blocks += nblk;
    quads += nquad;
  }
  return finish(launched(fp8q::launch_quant_weight_chunk(chunk, blocks, quads, pow2, s), "quant_weight_blk128"),
                stream, "quant_weight_blk128");
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
  if (debug_on()) {
    st = check_disjoint({extent(q, m, k, ld_q, "q"), extent(s, k / 128, 4 * m, 4 * ld_s, "s")},
                        {extent(x, m, 2 * k, 2 * ld_x, "x")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    if (st == FP8Q_OK) st = finite_bf16(x, m, k, ld_x, "x");
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_quant_act(x, m, k, ld_x, q, ld_q, s, ld_s, pow2,
                                                reinterpret_cast<hipStream_t>(stream)),
                         "quant_act_g128"),
                stream, "quant_act_g128");
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
  // the token scales are addressed as one [k/128][ld_as] fp32 range
  if (m * ld_a > kMaxOperandBytes || ld_as * 4 * (k / 128) > kMaxOperandBytes)
    return fail(FP8Q_ERR_SHAPE, "an operand spans more than 2 GiB (a, or a_s: 4 * ld_as * k/128 bytes)");
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
  if (debug_on()) {
    st = check_disjoint({extent(y, m, 2 * n, 2 * ld_y, "y")},
                        {extent(a, m, k, ld_a, "a"), extent(a_s, k / 128, 4 * m, 4 * ld_as, "a_s"),
                         extent(b, n, k, ld_b, "b"), extent(b_s, 1, (n / 128) * (k / 128) * 4, 0, "b_s")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    if (st == FP8Q_OK) st = no_nan_codes(a, m, k, ld_a, "a");
    if (st == FP8Q_OK) st = no_nan_codes(b, n, k, ld_b, "b");
    if (st == FP8Q_OK) st = check_f32(a_s, k / 128, m, ld_as, "a_s", pow2, false);
    if (st == FP8Q_OK) st = check_f32(b_s, n / 128, k / 128, k / 128, "b_s", pow2, false);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_gemm(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, pow2,
                                           reinterpret_cast<hipStream_t>(stream)),
                         "gemm_w8a8_blkscaled"),
                stream, "gemm_w8a8_blkscaled");
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

static fp8q_status gemm_bf16act(const void* x, int64_t ld_x, const void* b, int64_t ld_b, const float* b_s, void* y,
                                int64_t ld_y, int64_t m, int64_t n, int64_t k, void* stream, bool pow2) {
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
  if (debug_on()) {
    st = check_disjoint({extent(y, m, 2 * n, 2 * ld_y, "y")},
                        {extent(x, m, 2 * k, 2 * ld_x, "x"), extent(b, n, k, ld_b, "b"),
                         extent(b_s, 1, (n / 128) * (k / 128) * 4, 0, "b_s")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    if (st == FP8Q_OK) st = finite_bf16(x, m, k, ld_x, "x");
    if (st == FP8Q_OK) st = no_nan_codes(b, n, k, ld_b, "b");
    if (st == FP8Q_OK) st = check_f32(b_s, n / 128, k / 128, k / 128, "b_s", pow2, false);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_gemm_bf16act(x, ld_x, b, ld_b, b_s, y, ld_y, m, n, k, pow2,
                                                   reinterpret_cast<hipStream_t>(stream)),
                         "gemm_w8a8_bf16act"),
                stream, "gemm_w8a8_bf16act");
}

fp8q_status fp8q_gemm_w8a8_bf16act(const void* x, int64_t ld_x, const void* b, int64_t ld_b, const float* b_s,
                                   void* y, int64_t ld_y, int64_t m, int64_t n, int64_t k, void* stream) {
  return gemm_bf16act(x, ld_x, b, ld_b, b_s, y, ld_y, m, n, k, stream, false);
}

fp8q_status fp8q_gemm_w8a8_bf16act_ue8m0(const void* x, int64_t ld_x, const void* b, int64_t ld_b,
                                         const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n, int64_t k,
                                         void* stream) {
  return gemm_bf16act(x, ld_x, b, ld_b, b_s, y, ld_y, m, n, k, stream, true);
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
  if (debug_on()) {
    st = check_disjoint({extent(y, total_m, 2 * n, 2 * ld_y, "y")},
                        {extent(a, total_m, k, ld_a, "a"), extent(a_s, k / 128, 4 * total_m, 4 * ld_as, "a_s"),
                         extent(b, num_groups, n * k, n * k, "b"),
                         extent(b_s, num_groups, (n / 128) * (k / 128) * 4, (n / 128) * (k / 128) * 4, "b_s"),
                         extent(group_offsets, 1, 4 * ((int64_t)num_groups + 1), 0, "group_offsets")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    std::vector<int32_t> off;
    if (st == FP8Q_OK) st = fetch(off, group_offsets, 1, (int64_t)num_groups + 1, (int64_t)num_groups + 1);
    if (st == FP8Q_OK) {
      if (off[0] != 0) st = fail(FP8Q_ERR_PRECONDITION, "group_offsets[0] = %d, not 0", off[0]);
      for (int32_t g = 0; st == FP8Q_OK && g < num_groups; ++g)
        if (off[g + 1] < off[g])
          st = fail(FP8Q_ERR_PRECONDITION, "group_offsets decrease at %d (%d -> %d)", g, off[g], off[g + 1]);
      if (st == FP8Q_OK && off[num_groups] != total_m)
        st = fail(FP8Q_ERR_PRECONDITION, "group_offsets[%d] = %d, not total_m = %lld", num_groups, off[num_groups],
                  (long long)total_m);
    }
    if (st == FP8Q_OK) st = no_nan_codes(a, total_m, k, ld_a, "a");
    if (st == FP8Q_OK) st = no_nan_codes(b, num_groups * n, k, k, "b");
    if (st == FP8Q_OK) st = check_f32(a_s, k / 128, total_m, ld_as, "a_s", pow2, false);
    if (st == FP8Q_OK) st = check_f32(b_s, num_groups * (n / 128), k / 128, k / 128, "b_s", pow2, false);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_grouped_gemm(a, ld_a, a_s, ld_as, b, b_s, group_offsets, num_groups, total_m,
                                                   y, ld_y, n, k, pow2, reinterpret_cast<hipStream_t>(stream)),
                         "grouped_gemm_w8a8"),
                stream, "grouped_gemm_w8a8");
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

static fp8q_status grouped_swiglu(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                  const int32_t* row_token, int64_t token_rows, const void* b, const float* b_s,
                                  const int32_t* group_offsets, int32_t num_groups, int64_t total_m, void* q,
                                  int64_t ld_q, float* s, int64_t ld_s, int64_t n_half, int64_t k, void* stream,
                                  bool pow2) {
  if (num_groups < 1) return fail(FP8Q_ERR_SHAPE, "num_groups must be >= 1 (got %d)", num_groups);
  if (total_m < 0 || n_half < 0 || k < 0 || token_rows < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  const int64_t a_rows = row_token ? token_rows : total_m;  // rows of a (and columns of a_s)
  if (n_half == 0 || n_half % 128 || k == 0 || k % 128)
    return fail(FP8Q_ERR_SHAPE, "n_half=%lld and k=%lld must be positive multiples of 128", (long long)n_half,
                (long long)k);
  if (total_m > 0) {
    if (!a || !a_s || !b || !b_s || !group_offsets || !q || !s) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (row_token && token_rows < 1) return fail(FP8Q_ERR_SHAPE, "token_rows must be >= 1 with row_token");
    if (ld_a < k || ld_as < a_rows || ld_q < n_half || ld_s < total_m)
      return fail(FP8Q_ERR_STRIDE, "ld_a < k, ld_as < rows of a, ld_q < n_half or ld_s < total_m");
    if (!aligned16(a) || !aligned16(b) || !aligned16(q) || ld_a % 16 || ld_q % 16 || !aligned4(a_s) ||
        !aligned4(b_s) || !aligned4(s) || !aligned4(group_offsets) || !aligned4(row_token))
      return fail(FP8Q_ERR_ALIGN, "a/b/q must be 16-byte aligned with ld_a, ld_q multiples of 16");
    if (a_rows * ld_a > kMaxOperandBytes || ld_as * 4 * (k / 128) > kMaxOperandBytes ||
        2 * n_half * k > kMaxOperandBytes)
      return fail(FP8Q_ERR_SHAPE, "an operand spans more than 2 GiB (a, a_s: 4 * ld_as * k/128 bytes, or b)");
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  if (total_m == 0) return ok();
  if (debug_on()) {
    const int64_t bs_bytes = (2 * n_half / 128) * (k / 128) * 4;
    st = check_disjoint({extent(q, total_m, n_half, ld_q, "q"), extent(s, n_half / 128, 4 * total_m, 4 * ld_s, "s")},
                        {extent(a, a_rows, k, ld_a, "a"), extent(a_s, k / 128, 4 * a_rows, 4 * ld_as, "a_s"),
                         extent(row_token, 1, 4 * total_m, 0, "row_token"),
                         extent(b, num_groups, 2 * n_half * k, 2 * n_half * k, "b"),
                         extent(b_s, num_groups, bs_bytes, bs_bytes, "b_s"),
                         extent(group_offsets, 1, 4 * ((int64_t)num_groups + 1), 0, "group_offsets")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    std::vector<int32_t> off;
    if (st == FP8Q_OK) st = fetch(off, group_offsets, 1, (int64_t)num_groups + 1, (int64_t)num_groups + 1);
    if (st == FP8Q_OK) {
      if (off[0] != 0) st = fail(FP8Q_ERR_PRECONDITION, "group_offsets[0] = %d, not 0", off[0]);
      for (int32_t g = 0; st == FP8Q_OK && g < num_groups; ++g)
        if (off[g + 1] < off[g])
          st = fail(FP8Q_ERR_PRECONDITION, "group_offsets decrease at %d (%d -> %d)", g, off[g], off[g + 1]);
      if (st == FP8Q_OK && off[num_groups] != total_m)
        st = fail(FP8Q_ERR_PRECONDITION, "group_offsets[%d] = %d, not total_m = %lld", num_groups, off[num_groups],
                  (long long)total_m);
    }
    if (st == FP8Q_OK && row_token) {
      std::vector<int32_t> tokens;
      st = fetch(tokens, row_token, 1, total_m, total_m);
      for (int64_t r = 0; st == FP8Q_OK && r < total_m; ++r)
        if (tokens[r] < 0 || tokens[r] >= token_rows)
          st = fail(FP8Q_ERR_PRECONDITION, "row_token[%lld] = %d is not a row below token_rows = %lld",
                    (long long)r, tokens[r], (long long)token_rows);
    }
    if (st == FP8Q_OK) st = no_nan_codes(a, a_rows, k, ld_a, "a");
    if (st == FP8Q_OK) st = no_nan_codes(b, num_groups * 2 * n_half, k, k, "b");
    if (st == FP8Q_OK) st = check_f32(a_s, k / 128, a_rows, ld_as, "a_s", pow2, false);
    if (st == FP8Q_OK) st = check_f32(b_s, num_groups * (2 * n_half / 128), k / 128, k / 128, "b_s", pow2, false);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_grouped_swiglu(a, ld_a, a_s, ld_as, b, b_s, group_offsets, num_groups, total_m,
                                                     n_half, k, q, ld_q, s, ld_s, row_token, token_rows, pow2,
                                                     reinterpret_cast<hipStream_t>(stream)),
                         "grouped_gemm_swiglu_quant"),
                stream, "grouped_gemm_swiglu_quant");
}

fp8q_status fp8q_grouped_gemm_swiglu_quant(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                           const int32_t* row_token, int64_t token_rows, const void* b,
                                           const float* b_s, const int32_t* group_offsets, int32_t num_groups,
                                           int64_t total_m, void* q, int64_t ld_q, float* s, int64_t ld_s,
                                           int64_t n_half, int64_t k, void* stream) {
  return grouped_swiglu(a, ld_a, a_s, ld_as, row_token, token_rows, b, b_s, group_offsets, num_groups, total_m, q,
                        ld_q, s, ld_s, n_half, k, stream, false);
}

fp8q_status fp8q_grouped_gemm_swiglu_quant_ue8m0(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                                                 const int32_t* row_token, int64_t token_rows, const void* b,
                                                 const float* b_s, const int32_t* group_offsets,
                                                 int32_t num_groups, int64_t total_m, void* q, int64_t ld_q,
                                                 float* s, int64_t ld_s, int64_t n_half, int64_t k, void* stream) {
  return grouped_swiglu(a, ld_a, a_s, ld_as, row_token, token_rows, b, b_s, group_offsets, num_groups, total_m, q,
                        ld_q, s, ld_s, n_half, k, stream, true);
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
  if (debug_on()) {
    const bool recal = (flags & FP8Q_KV_RECALIBRATE) != 0;
    const int64_t cache_bytes = num_pages * page_size * row;
    std::vector<Extent> outs = {extent(k_cache, 1, cache_bytes, 0, "k_cache"),
                                extent(v_cache, 1, cache_bytes, 0, "v_cache")};
    std::vector<Extent> ins = {extent(k, num_tokens, 2 * row, 2 * ld_k, "k"), extent(v, num_tokens, 2 * row, 2 * ld_v, "v"),
                               extent(slot_mapping, 1, 8 * num_tokens, 0, "slot_mapping")};
    (recal ? outs : ins).push_back(extent(k_scale, 1, 4, 0, "k_scale"));
    (recal ? outs : ins).push_back(extent(v_scale, 1, 4, 0, "v_scale"));
    st = check_disjoint(outs, ins);
    if (st == FP8Q_OK) st = debug_sync(stream);
    std::vector<int64_t> slots;
    if (st == FP8Q_OK) st = fetch(slots, slot_mapping, 1, num_tokens, num_tokens);
    for (int64_t t = 0; st == FP8Q_OK && t < num_tokens; ++t)
      if (slots[t] >= num_pages * page_size)
        st = fail(FP8Q_ERR_PRECONDITION, "slot_mapping[%lld] = %lld is not below num_pages * page_size = %lld",
                  (long long)t, (long long)slots[t], (long long)(num_pages * page_size));
    if (st == FP8Q_OK) st = finite_bf16(k, num_tokens, row, ld_k, "k");
    if (st == FP8Q_OK) st = finite_bf16(v, num_tokens, row, ld_v, "v");
    if (st == FP8Q_OK && !recal) st = check_f32(k_scale, 1, 1, 1, "k_scale", false, true);
    if (st == FP8Q_OK && !recal) st = check_f32(v_scale, 1, 1, 1, "v_scale", false, true);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_kv_quant(k, ld_k, v, ld_v, num_tokens, num_kv_heads, slot_mapping, k_cache,
                                               v_cache, k_scale, v_scale, fp8_range,
                                               (flags & FP8Q_KV_RECALIBRATE) != 0,
                                               reinterpret_cast<hipStream_t>(stream)),
                         "kv_quant"),
                stream, "kv_quant");
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
  if (debug_on()) {
    st = check_disjoint({extent(aq, n, k, ld_aq, "aq"), extent(as, k / 128, 4 * n, 4 * ld_as, "as"),
                         extent(offsets, 1, 4 * ((int64_t)num_experts + 1), 0, "offsets"),
                         extent(row_of, 1, 4 * n, 0, "row_of")},
                        {extent(xq, num_tokens, k, ld_xq, "xq"), extent(xs, k / 128, 4 * num_tokens, 4 * ld_xs, "xs"),
                         extent(topk_ids, 1, 2 * n, 0, "topk_ids")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    if (st == FP8Q_OK && n > 0) st = no_nan_codes(xq, num_tokens, k, ld_xq, "xq");
    if (st == FP8Q_OK && n > 0) st = check_f32(xs, k / 128, num_tokens, ld_xs, "xs", false, false);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_moe_dispatch(xq, ld_xq, xs, ld_xs, topk_ids, num_tokens, topk, num_experts, k,
                                                   aq, ld_aq, as, ld_as, offsets, row_of,
                                                   reinterpret_cast<hipStream_t>(stream)),
                         "moe_dispatch"),
                stream, "moe_dispatch");
}

fp8q_status fp8q_moe_route(const int16_t* topk_ids, int64_t num_tokens, int32_t topk, int32_t num_experts,
                           int32_t* offsets, int32_t* row_of, int32_t* row_token, void* stream) {
  if (num_tokens < 0) return fail(FP8Q_ERR_SHAPE, "negative shape");
  if (topk < 1) return fail(FP8Q_ERR_SHAPE, "topk must be >= 1 (got %d)", topk);
  if (num_experts < 1 || num_experts > 32767)
    return fail(FP8Q_ERR_SHAPE, "num_experts must be in [1, 32767] (got %d)", num_experts);
  const int64_t n = num_tokens * (int64_t)topk;
  if (n > 0x7fffffffLL) return fail(FP8Q_ERR_SHAPE, "num_tokens * topk must be below 2^31");
  if (!offsets) return fail(FP8Q_ERR_NULL, "offsets is NULL");
  if (!aligned4(offsets)) return fail(FP8Q_ERR_ALIGN, "offsets must be 4-byte aligned");
  if (n > 0) {
    if (!topk_ids || !row_of || !row_token) return fail(FP8Q_ERR_NULL, "NULL pointer");
    if (!aligned16(topk_ids) || !aligned4(row_of) || !aligned4(row_token))
      return fail(FP8Q_ERR_ALIGN, "topk_ids must be 16-byte aligned, row_of and row_token 4-byte aligned");
  }
  fp8q_status st = check_device();
  if (st != FP8Q_OK) return st;
  if (debug_on()) {
    st = check_disjoint({extent(offsets, 1, 4 * ((int64_t)num_experts + 1), 0, "offsets"),
                         extent(row_of, 1, 4 * n, 0, "row_of"), extent(row_token, 1, 4 * n, 0, "row_token")},
                        {extent(topk_ids, 1, 2 * n, 0, "topk_ids")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_moe_route(topk_ids, num_tokens, topk, num_experts, offsets, row_of, row_token,
                                                reinterpret_cast<hipStream_t>(stream)),
                         "moe_route"),
                stream, "moe_route");
}

static fp8q_status swiglu_quant(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q, int64_t ld_q, float* s,
                                int64_t ld_s, void* stream, bool pow2) {
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
  if (debug_on()) {
    st = check_disjoint({extent(q, m, n, ld_q, "q"), extent(s, n / 128, 4 * m, 4 * ld_s, "s")},
                        {extent(h, m, 4 * n, 2 * ld_h, "h")});
    if (st == FP8Q_OK) st = debug_sync(stream);
    std::vector<uint16_t> hv;
    if (st == FP8Q_OK) st = fetch(hv, h, m, 2 * n, ld_h);
    auto dec = [](uint16_t b) {
      const uint32_t u = (uint32_t)b << 16;
      float f;
      std::memcpy(&f, &u, 4);
      return (double)f;
    };
    for (int64_t r = 0; st == FP8Q_OK && r < m; ++r)
      for (int64_t c = 0; st == FP8Q_OK && c < n; ++c) {
        const uint16_t gb = hv[r * 2 * n + c], ub = hv[r * 2 * n + n + c];
        if ((gb & 0x7f80u) == 0x7f80u || (ub & 0x7f80u) == 0x7f80u) {
          st = fail(FP8Q_ERR_PRECONDITION, "h[%lld][%lld] or its up value is not finite", (long long)r, (long long)c);
          break;
        }
        const double g = dec(gb), a = g / (1.0 + std::exp(-g)) * dec(ub);
        if (!pow2 && std::fabs(a) / 448.0 > 3.4028234663852886e38)
          st = fail(FP8Q_ERR_PRECONDITION, "silu(h[%lld][%lld]) * up = %g: its group's amax / 448 exceeds binary32",
                    (long long)r, (long long)c, a);
      }
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_swiglu_quant(h, m, n, ld_h, q, ld_q, s, ld_s, pow2,
                                                   reinterpret_cast<hipStream_t>(stream)),
                         "swiglu_quant_g128"),
                stream, "swiglu_quant_g128");
}

fp8q_status fp8q_swiglu_quant_g128(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q, int64_t ld_q,
                                   float* s, int64_t ld_s, void* stream) {
  return swiglu_quant(h, m, n, ld_h, q, ld_q, s, ld_s, stream, false);
}

fp8q_status fp8q_swiglu_quant_g128_ue8m0(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q, int64_t ld_q,
                                         float* s, int64_t ld_s, void* stream) {
  return swiglu_quant(h, m, n, ld_h, q, ld_q, s, ld_s, stream, true);
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
  if (debug_on()) {
    // y's rows are not passed: its extent is taken up to the largest row the call reads
    const int64_t entries = num_tokens * topk;
    st = debug_sync(stream);
    std::vector<int32_t> rows;
    if (st == FP8Q_OK) st = fetch(rows, row_of, 1, entries, entries);
    int64_t last = -1;
    for (int64_t i = 0; st == FP8Q_OK && i < entries; ++i) {
      if (rows[i] < -1)
        st = fail(FP8Q_ERR_PRECONDITION, "row_of[%lld] = %d is neither -1 nor a row", (long long)i, rows[i]);
      last = rows[i] > last ? rows[i] : last;
    }
    if (st == FP8Q_OK)
      st = check_disjoint({extent(out, num_tokens, 2 * hidden, 2 * ld_out, "out")},
                          {extent(y, last + 1, 2 * hidden, 2 * ld_y, "y"), extent(row_of, 1, 4 * entries, 0, "row_of"),
                           extent(weights, 1, 4 * entries, 0, "weights")});
    if (st == FP8Q_OK) st = check_f32(weights, 1, entries, entries, "weights", false, false);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_moe_combine(y, ld_y, row_of, weights, num_tokens, topk, hidden, out, ld_out,
                                                  reinterpret_cast<hipStream_t>(stream)),
                         "moe_combine"),
                stream, "moe_combine");
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
  if (debug_on()) {
    const bool recal = (flags & FP8Q_ATTN_RECALIBRATE_Q) != 0;
    const int64_t cache_bytes = num_pages * page_size * (int64_t)num_kv_heads * 128;
    std::vector<Extent> outs = {extent(out, num_seqs, 2 * row, 2 * ld_out, "out")};
    std::vector<Extent> ins = {extent(q, num_seqs, 2 * row, 2 * ld_q, "q"),
                               extent(k_cache, 1, cache_bytes, 0, "k_cache"),
                               extent(v_cache, 1, cache_bytes, 0, "v_cache"),
                               extent(block_table, num_seqs, 4 * ld_bt, 4 * ld_bt, "block_table"),
                               extent(seq_lens, 1, 4 * (int64_t)num_seqs, 0, "seq_lens"),
                               extent(k_scale, 1, 4, 0, "k_scale"), extent(v_scale, 1, 4, 0, "v_scale")};
    (recal ? outs : ins).push_back(extent(q_scale, 1, 4, 0, "q_scale"));
    st = check_disjoint(outs, ins);
    if (st == FP8Q_OK) st = debug_sync(stream);
    std::vector<int32_t> lens, table;
    if (st == FP8Q_OK) st = fetch(lens, seq_lens, 1, num_seqs, num_seqs);
    if (st == FP8Q_OK) st = fetch(table, block_table, num_seqs, ld_bt, ld_bt);
    for (int32_t b = 0; st == FP8Q_OK && b < num_seqs; ++b) {
      if (lens[b] < 0 || (int64_t)lens[b] > ld_bt * page_size) {
        st = fail(FP8Q_ERR_PRECONDITION, "seq_lens[%d] = %d is outside [0, ld_bt * page_size]", b, lens[b]);
        break;
      }
      const int64_t used = ((int64_t)lens[b] + page_size - 1) / page_size;
      for (int64_t i = 0; i < used; ++i) {
        const int32_t id = table[(size_t)b * ld_bt + i];
        if (id < 0 || id >= num_pages) {
          st = fail(FP8Q_ERR_PRECONDITION, "block_table[%d][%lld] = %d is not a page below num_pages = %lld", b,
                    (long long)i, id, (long long)num_pages);
          break;
        }
      }
    }
    if (st == FP8Q_OK) st = finite_bf16(q, num_seqs, row, ld_q, "q");
    if (st == FP8Q_OK) st = check_f32(k_scale, 1, 1, 1, "k_scale", false, true);
    if (st == FP8Q_OK) st = check_f32(v_scale, 1, 1, 1, "v_scale", false, true);
    if (st == FP8Q_OK && !recal) st = check_f32(q_scale, 1, 1, 1, "q_scale", false, true);
    if (st != FP8Q_OK) return st;
  }
  return finish(launched(fp8q::launch_decode_attention(q, ld_q, k_cache, v_cache, block_table, ld_bt, seq_lens,
                                                       num_seqs, num_q_heads, num_kv_heads, page_size, q_scale,
                                                       k_scale, v_scale, sm_scale, fp8_range,
                                                       (flags & FP8Q_ATTN_RECALIBRATE_Q) != 0, out, ld_out,
                                                       reinterpret_cast<hipStream_t>(stream)),
                         "paged_decode_attention"),
                stream, "paged_decode_attention");
}

}  // extern "C"

// The MoE layer's data movement around the grouped GEMM, for gfx950: dispatch of
// quantized tokens to their recorded experts, SwiGLU fused with fc2's 1x128
// quantization, and the weighted combine of the expert outputs.
//
// MoE routing-replay page, "Rollout Routing Replay" (section 4) and its cost analysis
// (section 5): the rollout records each token's top-k expert indices as int16 and the
// tokens go to exactly those experts.  Rounding-location page, the SwiGLU fusion
// region: SiLU's result is not rounded before it multiplies the up projection.
// FP8-RL summary page, "Method step details" step 1: MoE fc1/fc2 inputs are quantized
// per 1x128 group on every forward.
//
// All three are HBM streams.  Dispatch is deterministic without atomics: rows are
// ordered by expert and, within an expert, by entry index f = t*topk + j (a stable
// counting sort).
#include "e4m3.hpp"
#include "launch.hpp"
#include "swiglu.hpp"

namespace fp8q {

// ----------------------------------------------------------------------------
// Dispatch, routing step: one workgroup per expert e.  Each scans every recorded id
// twice.  Pass 1 counts the valid ids below e (the first row of e) and equal to e.
// Pass 2 hands the entries of e, in f order, consecutive rows: row_of[f] = row.
// Workgroup 0 also marks invalid entries (id < 0 or id >= E) with row -1.
// ----------------------------------------------------------------------------
constexpr int kRouteThreads = 1024;
constexpr int kRoutePer = 32;  // ids per thread and pass chunk: four 16-byte loads

// ids [f0, f0 + 64) of this thread (entries at or past n read as -1)
__device__ __forceinline__ void load_ids(const int16_t* __restrict__ ids, int64_t n, int64_t f0,
                                         int (&v)[kRoutePer]) {
  if (f0 + kRoutePer <= n) {
    uint4 w[kRoutePer / 8];
#pragma unroll
    for (int i = 0; i < kRoutePer / 8; ++i) w[i] = load_plain(ids + f0 + 8 * i);
#pragma unroll
    for (int i = 0; i < kRoutePer / 8; ++i) {
      const uint32_t d[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[8 * i + 2 * h] = (int)(int16_t)(d[h] & 0xffffu);
        v[8 * i + 2 * h + 1] = (int)(int16_t)(d[h] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kRoutePer; ++i) v[i] = (f0 + i < n) ? (int)ids[f0 + i] : -1;
  }
}

// Exclusive prefix of v over the workgroup in thread order; `total` gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kRouteThreads / 64; ++i) {
    const int s = sh[i];
    base += (i < w) ? s : 0;
    total += s;
  }
  __syncthreads();  // sh is reused by the next call
  return base + incl - v;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(const int16_t* __restrict__ ids, int64_t n,
                                                                   int32_t experts, int32_t* __restrict__ offsets,
                                                                   int32_t* __restrict__ row_of) {
  __shared__ int sh[kRouteThreads / 64];
  const int e = blockIdx.x;
  const int64_t chunk = (int64_t)kRouteThreads * kRoutePer;
  int v[kRoutePer];

  int below = 0, mine = 0;
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    load_ids(ids, n, c0 + (int64_t)threadIdx.x * kRoutePer, v);
#pragma unroll
    for (int i = 0; i < kRoutePer; ++i) {
      below += (v[i] >= 0 && v[i] < e) ? 1 : 0;
      mine += (v[i] == e) ? 1 : 0;
    }
  }
  int base, count;
  (void)block_excl_scan(below, sh, base);
  (void)block_excl_scan(mine, sh, count);
  if (threadIdx.x == 0) {
    offsets[e] = base;
    if (e == experts - 1) offsets[experts] = base + count;
  }

  int running = base;
  for (int64_t c0 = 0; c0 < n; c0 += chunk) {
    const int64_t f0 = c0 + (int64_t)threadIdx.x * kRoutePer;
    load_ids(ids, n, f0, v);
    uint64_t match = 0, bad = 0;
#pragma unroll
    for (int i = 0; i < kRoutePer; ++i) {
      match |= (uint64_t)(v[i] == e) << i;
      bad |= (uint64_t)(f0 + i < n && (v[i] < 0 || v[i] >= experts)) << i;
    }
    int tot;
    int r = running + block_excl_scan(__popcll(match), sh, tot);
    while (match) {
      row_of[f0 + __builtin_ctzll(match)] = r++;
      match &= match - 1;
    }
    if (e == 0) {
      while (bad) {
        row_of[f0 + __builtin_ctzll(bad)] = -1;
        bad &= bad - 1;
      }
    }
    running += tot;
  }
}

// ----------------------------------------------------------------------------
// Dispatch, copy step: one wave per entry copies the token's K code bytes into its row
// (up to 4 KB in flight before the first store) and its K/128 scales into column `row` of
// the dispatched scale matrix.
// ----------------------------------------------------------------------------
constexpr int kGatherWaves = 4;

__global__ __launch_bounds__(64 * kGatherWaves) void moe_gather_kernel(
    const uint8_t* __restrict__ xq, int64_t ld_xq, const float* __restrict__ xs, int64_t ld_xs,
    const int32_t* __restrict__ row_of, int64_t n, int32_t topk, int64_t k, uint8_t* __restrict__ aq,
    int64_t ld_aq, float* __restrict__ as, int64_t ld_as) {
  const int lane = threadIdx.x & 63;
  const int64_t f = (int64_t)blockIdx.x * kGatherWaves + (threadIdx.x >> 6);
  if (f >= n) return;
  const int32_t r = row_of[f];
  if (r < 0) return;
  const int64_t t = f / topk;
  const uint8_t* src = xq + t * ld_xq;
  uint8_t* dst = aq + (int64_t)r * ld_aq;
  // up to 4 KB of the row in flight before the first store
  for (int64_t c0 = (int64_t)lane * 16; c0 < k; c0 += 4 * 64 * 16) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + u * 64 * 16;
      v[u] = c < k ? load_plain(src + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t c = c0 + u * 64 * 16;
      if (c < k) store_plain(dst + c, v[u]);
    }
  }
  for (int64_t g = lane; g < k / 128; g += 64) as[g * ld_as + r] = xs[g * ld_xs + t];
}

hipError_t launch_moe_dispatch(const void* xq, int64_t ld_xq, const float* xs, int64_t ld_xs, const int16_t* ids,
                               int64_t tokens, int32_t topk, int32_t experts, int64_t k, void* aq, int64_t ld_aq,
                               float* as, int64_t ld_as, int32_t* offsets, int32_t* row_of, hipStream_t stream) {
  const int64_t n = tokens * topk;
  hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)experts), dim3(kRouteThreads), 0, stream, ids, n, experts,
                     offsets, row_of);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n == 0) return err;
  hipLaunchKernelGGL(moe_gather_kernel, dim3((unsigned)((n + kGatherWaves - 1) / kGatherWaves)),
                     dim3(64 * kGatherWaves), 0, stream, reinterpret_cast<const uint8_t*>(xq), ld_xq, xs, ld_xs,
                     row_of, n, topk, k, reinterpret_cast<uint8_t*>(aq), ld_aq, as, ld_as);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// SwiGLU + 1x128 quantization, standalone: h = [gate | up], bf16 [m, 2n].  8 lanes per
// (row, 128-column group), 16 values each (the activation quantizer's lane mapping); the
// arithmetic is swiglu_quant16 (swiglu.hpp), which the fc1 GEMM's fused epilogue shares.
// ----------------------------------------------------------------------------
template <bool POW2>
__global__ __launch_bounds__(256) void swiglu_quant_g128_kernel(const uint16_t* __restrict__ h, int64_t m,
                                                                int64_t groups, int64_t n, int64_t ld_h,
                                                                uint8_t* __restrict__ q, int64_t ld_q,
                                                                float* __restrict__ s, int64_t ld_s,
                                                                int64_t group_tiles) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t rb = blockIdx.x / group_tiles;
  const int64_t g = (blockIdx.x - rb * group_tiles) * 4 + wave;
  const int64_t row = rb * 8 + (lane >> 3);
  const int col = (lane & 7) * 16;
  const bool live = (g < groups) && (row < m);
  uint4 ga = make_uint4(0, 0, 0, 0), gb = ga, ua = ga, ub = ga;
  if (live) {
    const uint16_t* p = h + row * ld_h + g * 128 + col;
    ga = load_plain(p);
    gb = load_plain(p + 8);
    ua = load_plain(p + n);
    ub = load_plain(p + n + 8);
  }
  const uint32_t gw[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
  const uint32_t uw[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};

  uint32_t o[4];
  float scale;
  if (!swiglu_quant16<POW2>(gw, uw, live, o, scale)) return;
  if ((lane & 7) == 0) s[g * ld_s + row] = scale;
  store_plain(q + row * ld_q + g * 128 + col, make_uint4(o[0], o[1], o[2], o[3]));
}

// The inverse of row_of, for GEMMs that read each dispatched row straight from the token
// matrix: row_token[row_of[f]] = f / topk (f < 2^31), one thread per entry.
__global__ __launch_bounds__(256) void moe_row_token_kernel(const int32_t* __restrict__ row_of, int32_t n,
                                                            int32_t topk, int32_t* __restrict__ row_token) {
  const int32_t f = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (f >= n) return;
  const int32_t r = row_of[f];
  if (r >= 0) row_token[r] = (int32_t)((uint32_t)f / (uint32_t)topk);
}

hipError_t launch_moe_route(const int16_t* ids, int64_t tokens, int32_t topk, int32_t experts, int32_t* offsets,
                            int32_t* row_of, int32_t* row_token, hipStream_t stream) {
  const int64_t n = tokens * topk;
  hipLaunchKernelGGL(moe_route_kernel, dim3((unsigned)experts), dim3(kRouteThreads), 0, stream, ids, n, experts,
                     offsets, row_of);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || n == 0) return err;
  hipLaunchKernelGGL(moe_row_token_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, row_of,
                     (int32_t)n, topk, row_token);
  return hipGetLastError();
}

hipError_t launch_swiglu_quant(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q, int64_t ld_q, float* s,
                               int64_t ld_s, bool pow2, hipStream_t stream) {
  const int64_t groups = n / 128;
  const int64_t group_tiles = (groups + 3) / 4;
  const int64_t wgs = ((m + 7) / 8) * group_tiles;
  auto kernel = pow2 ? swiglu_quant_g128_kernel<true> : swiglu_quant_g128_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(256), 0, stream,
                     reinterpret_cast<const uint16_t*>(h), m, groups, n, ld_h, reinterpret_cast<uint8_t*>(q), ld_q,
                     s, ld_s, group_tiles);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Combine: out[t] = bf16( sum_j w[t, j] * y[row_of[t, j]] ), the sum in fp32 in the
// order j = 0, 1, ... (one FMA per term), entries with row -1 skipped, one rounding to
// bf16 at the store.  One wave per (token, 512-column block); each lane takes 8
// consecutive columns and has the up-to-8 expert rows of its columns in flight at once,
// so a wave makes a single round trip (a wave per token walking its columns in passes
// waits on each pass in turn).
// ----------------------------------------------------------------------------
constexpr int kCombineWaves = 4;
constexpr int kCombineBatch = 8;  // expert rows loaded together

__device__ __forceinline__ uint32_t bf16_pack_rne(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a = (a + 0x7fffu + ((a >> 16) & 1u)) >> 16;
  b = (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
  return a | (b << 16);
}

__global__ __launch_bounds__(64 * kCombineWaves) void moe_combine_kernel(
    const uint16_t* __restrict__ y, int64_t ld_y, const int32_t* __restrict__ row_of, const float* __restrict__ w,
    int64_t tokens, int32_t topk, int64_t hidden, uint16_t* __restrict__ out, int64_t ld_out) {
  const int lane = threadIdx.x & 63;
  // one wave per (token, 512-column block): a single round trip of loads per wave
  const int64_t cblocks = (hidden + 64 * 8 - 1) / (64 * 8);
  const int64_t f = (int64_t)blockIdx.x * kCombineWaves + (threadIdx.x >> 6);
  if (f >= tokens * cblocks) return;
  const int64_t t = f / cblocks;
  const int32_t* rt = row_of + t * topk;
  const float* wt = w + t * topk;
  {
    const int64_t c = (f - t * cblocks) * 64 * 8 + (int64_t)lane * 8;
    if (c >= hidden) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < topk; j0 += kCombineBatch) {
      uint4 v[kCombineBatch];
      float wj[kCombineBatch];
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        const int32_t r = (j0 + j < topk) ? rt[j0 + j] : -1;
        wj[j] = (r >= 0) ? wt[j0 + j] : 0.0f;
        v[j] = (r >= 0) ? load_plain(y + (int64_t)r * ld_y + c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kCombineBatch; ++j) {
        if (j0 + j >= topk || rt[j0 + j] < 0) continue;
        const uint32_t d[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = __builtin_fmaf(wj[j], bf16_lo(d[i]), acc[2 * i]);
          acc[2 * i + 1] = __builtin_fmaf(wj[j], bf16_hi(d[i]), acc[2 * i + 1]);
        }
      }
    }
    store_plain(out + t * ld_out + c, make_uint4(bf16_pack_rne(acc[0], acc[1]), bf16_pack_rne(acc[2], acc[3]),
                                                 bf16_pack_rne(acc[4], acc[5]), bf16_pack_rne(acc[6], acc[7])));
  }
}

hipError_t launch_moe_combine(const void* y, int64_t ld_y, const int32_t* row_of, const float* w, int64_t tokens,
                              int32_t topk, int64_t hidden, void* out, int64_t ld_out, hipStream_t stream) {
  const int64_t waves = tokens * ((hidden + 64 * 8 - 1) / (64 * 8));
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)((waves + kCombineWaves - 1) / kCombineWaves)),
                     dim3(64 * kCombineWaves), 0, stream, reinterpret_cast<const uint16_t*>(y), ld_y, row_of, w,
                     tokens, topk, hidden, reinterpret_cast<uint16_t*>(out), ld_out);
  return hipGetLastError();
}

}  // namespace fp8q

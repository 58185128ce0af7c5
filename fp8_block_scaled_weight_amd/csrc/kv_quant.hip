// FP8 KV-cache quantize-on-write with per-step K/V scale recalibration, gfx950.
//
// FP8-RL summary page, "Method step details" step 3: the KV cache is stored in FP8
// and its K/V scales are recomputed from the data at the start of every RL step's
// rollout.  "1T-parameter RL on 100 GPUs", 3.4: the cache is paged in fixed blocks
// and K and V are quantized to FP8 separately.
//
// Recalibration is a global dependency (every code needs the final amax), so a
// recalibrating call is two streaming passes: an amax pass (2 B/element read) and an
// encode pass (2 B read + 1 B written per element).  The amax is accumulated in the
// scale slot itself as 0x80000000 | bits(amax) with an unsigned atomic max: exact,
// order-independent, and marked as "not yet a scale" by the sign bit.  The encode
// pass turns a marked value into the scale in every workgroup (all get the same
// number) and workgroup 0 stores it back, so a workgroup reads either the marked amax
// or the final scale and derives the same scale from both.
#include "e4m3.hpp"
#include "launch.hpp"

namespace fp8q {

constexpr int kKvBlock = 256;                 // encode pass: 4 waves
constexpr int kKvAmaxBlock = 1024;            // amax pass: 16 waves
constexpr int kElemsPerWavePass = 64 * 16;    // 64 lanes x 16 bf16
constexpr uint32_t kMarked = 0x80000000u;
constexpr int kKvTokensInFlight = 1;          // encode pass: token rows loaded together per wave

__global__ void kv_reset_kernel(float* k_scale, float* v_scale) {
  if (threadIdx.x == 0) {
    reinterpret_cast<uint32_t*>(k_scale)[0] = kMarked;  // marked amax 0
    reinterpret_cast<uint32_t*>(v_scale)[0] = kMarked;
  }
}

// One wave per token (grid-stride), two tokens in flight per wave; one atomic per
// tensor per workgroup.  Few, wide workgroups keep the number of same-address atomics
// small: they are performed past the per-XCD L2s and serialize there.  Lane l reads
// elements 8l .. 8l+7 and 512 + 8l .. of each 1024-element pass of a row, so that every
// load instruction covers 1 KB contiguous (64 x 20,000-token layer: this pass 817 ->
// 781 us against 32 contiguous bytes per lane, i.e. 16 lanes' loads spanning 512 bytes
// with gaps).
__global__ __launch_bounds__(kKvAmaxBlock) void kv_amax_kernel(const uint16_t* __restrict__ k, int64_t ld_k,
                                                               const uint16_t* __restrict__ v, int64_t ld_v,
                                                               int64_t tokens, int64_t row,
                                                               const int64_t* __restrict__ slots,
                                                               float* k_scale, float* v_scale) {
  constexpr int W = kKvAmaxBlock / 64;
  __shared__ uint32_t red[2][W];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t waves = (int64_t)gridDim.x * W;
  uint32_t mk = 0, mv = 0;
  auto token = [&](int64_t t) {
    if (slots[t] < 0) return;  // uniform per wave
    for (int64_t e0 = 0; e0 < row; e0 += kElemsPerWavePass) {
      const int64_t ea = e0 + lane * 8, eb = ea + kElemsPerWavePass / 2;
      if (ea < row) {
        mk = max(mk, absmax8(load_plain(k + t * ld_k + ea)));
        mv = max(mv, absmax8(load_plain(v + t * ld_v + ea)));
      }
      if (eb < row) {
        mk = max(mk, absmax8(load_plain(k + t * ld_k + eb)));
        mv = max(mv, absmax8(load_plain(v + t * ld_v + eb)));
      }
    }
  };
  int64_t t = (int64_t)blockIdx.x * W + wave;
  for (; t + waves < tokens; t += 2 * waves) {
    token(t);
    token(t + waves);
  }
  if (t < tokens) token(t);
  mk = max_over_wave(mk);
  mv = max_over_wave(mv);
  if (lane == 0) {
    red[0][wave] = mk;
    red[1][wave] = mv;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0, b = 0;
    for (int w = 0; w < W; ++w) {
      a = max(a, red[0][w]);
      b = max(b, red[1][w]);
    }
    // the bf16 magnitude bits shifted up are the fp32 bits of the magnitude
    if (a) atomicMax(reinterpret_cast<unsigned int*>(k_scale), kMarked | (a << 16));
    if (b) atomicMax(reinterpret_cast<unsigned int*>(v_scale), kMarked | (b << 16));
  }
}

// The scale a slot stands for: a marked amax becomes fl32(amax / range) (1 for 0).
__device__ __forceinline__ float resolve_scale(uint32_t bits, float range) {
  return (bits & kMarked) ? scale_from_amax(__uint_as_float(bits & ~kMarked), range) : __uint_as_float(bits);
}

// One wave per token: K row then V row, in the amax pass's lane layout (each load
// instruction 1 KB contiguous, each code store 512 bytes).  Loads are non-temporal here
// (measured faster for this pass), plain in the amax pass.  Against 16 contiguous
// elements per lane the recalibrating call measured 2.32 -> 2.28-2.29 ms (64 x 20,000
// tokens; this pass alone unchanged).
__global__ __launch_bounds__(kKvBlock) void kv_write_kernel(const uint16_t* __restrict__ k, int64_t ld_k,
                                                            const uint16_t* __restrict__ v, int64_t ld_v,
                                                            int64_t tokens, int64_t row,
                                                            const int64_t* __restrict__ slots,
                                                            uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                            float* k_scale, float* v_scale, float range) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t waves = (int64_t)gridDim.x * (kKvBlock / 64);
  const float sk = resolve_scale(__atomic_load_n(reinterpret_cast<uint32_t*>(k_scale), __ATOMIC_RELAXED), range);
  const float sv = resolve_scale(__atomic_load_n(reinterpret_cast<uint32_t*>(v_scale), __ATOMIC_RELAXED), range);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    __atomic_store_n(reinterpret_cast<uint32_t*>(k_scale), __float_as_uint(sk), __ATOMIC_RELAXED);
    __atomic_store_n(reinterpret_cast<uint32_t*>(v_scale), __float_as_uint(sv), __ATOMIC_RELAXED);
  }
  const Quantizer qk = make_quantizer(sk);
  const Quantizer qv = make_quantizer(sv);
  // kKvTokensInFlight tokens per wave: every row's loads are issued before any is encoded
  constexpr int NT = kKvTokensInFlight;
  for (int64_t t0 = (int64_t)blockIdx.x * (kKvBlock / 64) + wave; t0 < tokens; t0 += NT * waves) {
    int64_t sl[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) sl[u] = (t0 + u * waves < tokens) ? slots[t0 + u * waves] : -1;
    // the amax pass's lane layout: elements 8l .. and 512 + 8l .. of each 1024-element pass;
    // each store instruction writes 8 codes per lane, a 512-byte run
    for (int64_t e0 = 0; e0 < row; e0 += kElemsPerWavePass) {
      const int64_t ea = e0 + lane * 8, eb = ea + kElemsPerWavePass / 2;
      const bool va = ea < row, vb = eb < row;
      uint4 x[NT][4];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        if (sl[u] >= 0) {  // uniform per wave
          const int64_t t = t0 + u * waves;
          if (va) {
            x[u][0] = load_stream(k + t * ld_k + ea);
            x[u][2] = load_stream(v + t * ld_v + ea);
          }
          if (vb) {
            x[u][1] = load_stream(k + t * ld_k + eb);
            x[u][3] = load_stream(v + t * ld_v + eb);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        if (sl[u] < 0) continue;
        if (va) {
          store8_stream(kc + sl[u] * row + ea, quant8<true>(x[u][0], qk, qk.xm != 1.0f));
          store8_stream(vc + sl[u] * row + ea, quant8<true>(x[u][2], qv, qv.xm != 1.0f));
        }
        if (vb) {
          store8_stream(kc + sl[u] * row + eb, quant8<true>(x[u][1], qk, qk.xm != 1.0f));
          store8_stream(vc + sl[u] * row + eb, quant8<true>(x[u][3], qv, qv.xm != 1.0f));
        }
      }
    }
  }
}

static unsigned kv_grid(int64_t tokens) {
  // up to one wave per token, at most 256 workgroups per CU's worth: a 64 x 20,000-token layer
  // then gives each wave about 5 tokens.  Measured on that layer (encode pass alone, with
  // interleaved builds): 16 workgroups per CU and two tokens in flight per wave 1.58 ms,
  // 64 / 128 / 256 per CU 1.55 / 1.54 / 1.52 ms, 256 with one token in flight 1.51 ms; one
  // wave per token (320,000 workgroups) 1.67 ms.
  int64_t wgs = (tokens + 3) / 4;
  const int64_t cap = 256 * 256;
  return (unsigned)(wgs < cap ? (wgs < 1 ? 1 : wgs) : cap);
}

static unsigned kv_amax_grid(int64_t tokens) {
  // one wave per token up to 256 workgroups of 16 waves
  const int64_t wgs = (tokens + 15) / 16;
  return (unsigned)(wgs < 256 ? (wgs < 1 ? 1 : wgs) : 256);
}

hipError_t launch_kv_quant(const void* k, int64_t ld_k, const void* v, int64_t ld_v, int64_t tokens,
                           int32_t heads, const int64_t* slots, void* k_cache, void* v_cache,
                           float* k_scale, float* v_scale, float range, bool recalibrate,
                           hipStream_t stream) {
  const int64_t row = (int64_t)heads * 128;
  const unsigned grid = kv_grid(tokens);
  const uint16_t* kk = reinterpret_cast<const uint16_t*>(k);
  const uint16_t* vv = reinterpret_cast<const uint16_t*>(v);
  if (recalibrate) {
    hipLaunchKernelGGL(kv_reset_kernel, dim3(1), dim3(64), 0, stream, k_scale, v_scale);
    hipLaunchKernelGGL(kv_amax_kernel, dim3(kv_amax_grid(tokens)), dim3(kKvAmaxBlock), 0, stream, kk, ld_k, vv,
                       ld_v, tokens, row, slots, k_scale, v_scale);
  }
  hipLaunchKernelGGL(kv_write_kernel, dim3(grid), dim3(kKvBlock), 0, stream, kk, ld_k, vv, ld_v, tokens, row,
                     slots, reinterpret_cast<uint8_t*>(k_cache), reinterpret_cast<uint8_t*>(v_cache),
                     k_scale, v_scale, range);
  return hipGetLastError();
}

}  // namespace fp8q

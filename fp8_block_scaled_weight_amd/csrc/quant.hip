// Blockwise weight quantization (128x128 blocks) and dynamic 1x128 activation
// quantization for gfx950.
//
// FP8-RL summary page: "Prerequisites / FP8 quantization format" (one scale per
// 128x128 block, W_hat = round(W / scale)), "Method step details" step 1 (weights
// quantized statically at every sync, activations dynamically on every forward)
// and step 2 (the sync quantizes every linear of every layer).
//
// Both kernels are single-pass HBM streams: each bf16 element is read once, kept in
// registers while the block/group amax is reduced, and written once as an E4M3 byte.
// Loads are plain (measured faster than non-temporal loads for this 2:1 read/write
// mix); the weight codes are stored non-temporally (the sync writes gigabytes that no
// kernel reads right away), the activation codes plainly (the GEMM reads them next).
#include "e4m3.hpp"
#include "launch.hpp"

namespace fp8q {

// POW2 selects the power-of-two (UE8M0) scale variant of the same quantizers (FP8-RL
// summary page, "Experimental results": the scale-format ablation); the encoding is the
// same, and with a power-of-two scale the quotient it rounds is exact.
//
// ----------------------------------------------------------------------------
// Weights: one 256-thread workgroup per 128x128 block.  Thread t covers columns
// 16*(t%8) .. +15 of rows t/8 + 32*i (i < 4): 8 x 16-byte loads, 4 x 16-byte stores.
// A launch covers a chunk of descriptors; block ids are laid out descriptor after
// descriptor, row-major over the block grid of each.
// ----------------------------------------------------------------------------
template <bool POW2>
__global__ __launch_bounds__(256) void quant_weight_blk128_kernel(WeightChunk chunk) {
  __shared__ uint32_t wave_max[4];
  const int64_t blk = blockIdx.x;
  // descriptor lookup: largest d with first_block[d] <= blk (uniform)
  int lo = 0, hi = chunk.count - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (chunk.d[mid].first_block <= blk) lo = mid; else hi = mid - 1;
  }
  const WeightDescDev& d = chunk.d[lo];
  const int64_t local = blk - d.first_block;
  const int64_t bi = local / d.kblocks;
  const int64_t bj = local - bi * d.kblocks;

  const int t = threadIdx.x;
  const int col = (t & 7) * 16;
  const int row0 = t >> 3;
  const uint16_t* w = reinterpret_cast<const uint16_t*>(d.w) + (bi * 128) * d.ld_w + bj * 128 + col;
  uint8_t* q = reinterpret_cast<uint8_t*>(d.q) + (bi * 128) * d.ld_q + bj * 128 + col;

  uint4 v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4* p = reinterpret_cast<const uint4*>(w + (int64_t)(row0 + 32 * i) * d.ld_w);
    v[2 * i] = load_plain(p);
    v[2 * i + 1] = load_plain(p + 1);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, absmax16(v[2 * i], v[2 * i + 1]));
  m = max_over_wave(m);
  if ((t & 63) == 0) wave_max[t >> 6] = m;
  __syncthreads();
  m = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  const float scale = block_scale<POW2>(bf16_bits_to_float(m), kE4M3Max);
  if (t == 0) d.s[bi * d.kblocks + bj] = scale;
  const Quantizer qz = make_quantizer(scale);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 o = quant16<false>(v[2 * i], v[2 * i + 1], qz);
    store_stream(q + (int64_t)(row0 + 32 * i) * d.ld_q, o);
  }
}

// Large launches: one 512-thread workgroup per four blocks side by side in a block row,
// so every row is read and written in 1 KB runs instead of 256-byte ones.  Thread t covers
// columns 16*(t%32) .. +15 of the four blocks' 512 (block (t%32)/8) in rows t/32 + 16*i
// (i < 8).  A block's amax: 8 lanes of a row, the two rows of a wave, then the 8 waves
// through LDS.  A block row's last workgroup may hold fewer than four blocks; its other
// lanes load and store nothing.
template <bool POW2>
__global__ __launch_bounds__(512) void quant_weight_blk128x4_kernel(WeightChunk chunk) {
  __shared__ uint32_t wave_max[8][4];
  const int64_t wg = blockIdx.x;
  int lo = 0, hi = chunk.count - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (chunk.d[mid].first_quad <= wg) lo = mid; else hi = mid - 1;
  }
  const WeightDescDev& d = chunk.d[lo];
  const int64_t local = wg - d.first_quad;
  const int64_t bi = local / d.kquads;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int c = t & 31, b = c >> 3;
  const int64_t bj = (local - bi * d.kquads) * 4 + b;
  const bool live = bj < d.kblocks;  // uniform over 8 lanes of a row
  const int col = (c & 7) * 16;
  const int row0 = t >> 5;
  const uint16_t* w = reinterpret_cast<const uint16_t*>(d.w) + (bi * 128) * d.ld_w + bj * 128 + col;
  uint8_t* q = reinterpret_cast<uint8_t*>(d.q) + (bi * 128) * d.ld_q + bj * 128 + col;

  uint4 v[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (live) {
      const uint4* p = reinterpret_cast<const uint4*>(w + (int64_t)(row0 + 16 * i) * d.ld_w);
      v[2 * i] = load_plain(p);
      v[2 * i + 1] = load_plain(p + 1);
    } else {
      v[2 * i] = v[2 * i + 1] = make_uint4(0, 0, 0, 0);
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, absmax16(v[2 * i], v[2 * i + 1]));
  m = max_over_8_lanes(m);
  m = max(m, (uint32_t)__shfl_xor((int)m, 32));
  if ((lane & 39) == 0) wave_max[wave][b] = m;  // lanes 0, 8, 16, 24: blocks 0..3
  __syncthreads();
  m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, wave_max[i][b]);
  const float scale = block_scale<POW2>(bf16_bits_to_float(m), kE4M3Max);
  if (!live) return;
  if (t < 32 && (t & 7) == 0) d.s[bi * d.kblocks + bj] = scale;
  const Quantizer qz = make_quantizer(scale);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    store_stream(q + (int64_t)(row0 + 16 * i) * d.ld_q, quant16<false>(v[2 * i], v[2 * i + 1], qz));
}

hipError_t launch_quant_weight_chunk(const WeightChunk& chunk, int64_t blocks, int64_t quads, bool pow2,
                                     hipStream_t stream) {
  // four blocks per workgroup once a launch moves 1 GB or more (48 KB of traffic per block)
#ifndef WIDE_MIN_BLOCKS
#define WIDE_MIN_BLOCKS 21846
#endif
  if (blocks >= WIDE_MIN_BLOCKS) {
    if (pow2)
      hipLaunchKernelGGL(quant_weight_blk128x4_kernel<true>, dim3((unsigned)quads), dim3(512), 0, stream, chunk);
    else
      hipLaunchKernelGGL(quant_weight_blk128x4_kernel<false>, dim3((unsigned)quads), dim3(512), 0, stream, chunk);
    return hipGetLastError();
  }
  if (pow2)
    hipLaunchKernelGGL(quant_weight_blk128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, chunk);
  else
    hipLaunchKernelGGL(quant_weight_blk128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, chunk);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Activations: 8 lanes per 1x128 group, 16 elements per lane.  A wave takes the
// same group g of 8 consecutive rows, so its 8 scales s[g*ld_s + r .. r+7] form one
// contiguous 32-byte store; the 4 waves of a workgroup take 4 consecutive row blocks
// of the same group, so together they write one 128-byte run of scales (measured with
// every call's buffers outside the caches: 32768 x 768, 22.1 -> 18.7 us against 4
// consecutive groups per workgroup; 4096 x 4096 and 4096 x 12288 unchanged).
// ----------------------------------------------------------------------------
template <bool POW2>
__global__ __launch_bounds__(256) void quant_act_g128_kernel(const uint16_t* __restrict__ x, int64_t m,
                                                             int64_t groups, int64_t ld_x,
                                                             uint8_t* __restrict__ q, int64_t ld_q,
                                                             float* __restrict__ s, int64_t ld_s) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // workgroup -> (4 row blocks of 8, one group)
  const int64_t rb = (blockIdx.x / groups) * 4 + wave;
  const int64_t g = blockIdx.x % groups;
  const int64_t row = rb * 8 + (lane >> 3);
  const int col = (lane & 7) * 16;
  const bool live = row < m;
  uint4 a = make_uint4(0, 0, 0, 0), b = a;
  if (live) {
    const uint4* p = reinterpret_cast<const uint4*>(x + row * ld_x + g * 128 + col);
    a = load_plain(p);
    b = load_plain(p + 1);
  }
  uint32_t mx = max_over_8_lanes(absmax16(a, b));
  if (!live) return;
  const float scale = block_scale<POW2>(bf16_bits_to_float(mx), kE4M3Max);
  if ((lane & 7) == 0) s[g * ld_s + row] = scale;
  const Quantizer qz = make_quantizer(scale);
  uint4 o = quant16<false>(a, b, qz);
  store_plain(q + row * ld_q + g * 128 + col, o);
}

hipError_t launch_quant_act(const void* x, int64_t m, int64_t k, int64_t ld_x, void* q, int64_t ld_q,
                            float* s, int64_t ld_s, bool pow2, hipStream_t stream) {
  const int64_t groups = k / 128;
  const int64_t row_quads = (m + 31) / 32;  // 4 row blocks of 8 per workgroup
  const int64_t wgs = row_quads * groups;
  auto kernel = pow2 ? quant_act_g128_kernel<true> : quant_act_g128_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)wgs), dim3(256), 0, stream, reinterpret_cast<const uint16_t*>(x), m,
                     groups, ld_x, reinterpret_cast<uint8_t*>(q), ld_q, s, ld_s);
  return hipGetLastError();
}

}  // namespace fp8q

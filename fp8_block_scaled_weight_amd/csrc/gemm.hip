// Block-scaled W8A8 GEMM, dense and MoE-grouped, for gfx950.
//
// FP8-RL summary page, "Method step details" step 1: linears run with FP8 weights
// (one fp32 scale per 128x128 block) and FP8 activations quantized per forward (one
// fp32 scale per 1x128 token group).  "Where rounding happens matters": all scaling
// and accumulation stay in fp32 and the output is rounded to bf16 once.
//
//   y[m, n] = bf16( sum_kb  sa[kb][m] * sb[n/128][kb] * P_kb[m, n] ),
//   P_kb[m, n] = sum_{k in block kb} a[m, k] * b[n, k]   (FP8 x FP8, fp32 accumulate)
//
// Each 128-wide K block is exactly one v_mfma_f32_16x16x128_f8f6f4 per 16x16 output
// tile, started from a zero accumulator, so P_kb comes out of the matrix core whole
// and is folded into the running fp32 sum with one FMA per element (the "promotion").
//
// Operand roles: the MFMA's A operand is 16 weight rows (n) and its B operand 16
// activation rows (m); both are K-contiguous, so both fragments are loaded the same
// way (lane l: row l%16, 32 bytes at K offset 32*(l/16)) and any K order the matrix
// core uses internally applies to both.  The 16x16 result then has lane l holding
// m = l%16 and n = 4*(l/16) + r, r = 0..3: four consecutive outputs of one row
// (an 8-byte store) and a single activation scale per lane and tile.
//
// Tiles: a 256-thread workgroup computes BN x BM outputs (weights x tokens) with 4
// waves in a 2 x 2 grid; per K step both 128-byte-wide operand tiles are staged in
// LDS, double-buffered.  LDS rows are 128 bytes; the 16-byte chunk c of row r is
// stored at chunk c ^ (r & 7) so that 8 consecutive rows read at the same K offset
// hit 8 different bank groups.
#include "launch.hpp"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  v4f zero = {0.f, 0.f, 0.f, 0.f};
  // scale operands 0 select the unscaled FP8 x FP8 -> fp32 instruction
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int WN, int WM>  // MFMA tiles per wave along n and m
struct TileCfg {
  static constexpr int kWavesN = 2, kWavesM = 2;
  static constexpr int BN = kWavesN * WN * 16;
  static constexpr int BM = kWavesM * WM * 16;
  static constexpr int kThreads = 256;
  static constexpr int kTileBytesA = BN * 128;  // weights
  static constexpr int kTileBytesB = BM * 128;  // activations
  static constexpr int kLoadsA = kTileBytesA / (16 * kThreads);
  static constexpr int kLoadsB = kTileBytesB / (16 * kThreads);
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

// One output tile: rows [m0, m0+BM) of a (clipped to m_end), columns [n0, n0+BN).
// b points at the weight matrix of this tile's group ([n][k]), bs at its scales.
template <int WN, int WM>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ a, int64_t ld_a,
                                          const float* __restrict__ as, int64_t ld_as,
                                          const uint8_t* __restrict__ b, int64_t ld_b,
                                          const float* __restrict__ bs, uint16_t* __restrict__ y,
                                          int64_t ld_y, int64_t m0, int64_t m_end, int64_t n0,
                                          int64_t kblocks, uint8_t* lds) {
  using C = TileCfg<WN, WM>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = (wave % C::kWavesN) * WN * 16;  // wave offset along n within the tile
  const int wm = (wave / C::kWavesN) * WM * 16;  // wave offset along m

  // LDS stage s (s = 0, 1) holds the weight tile then the activation tile
  constexpr int kStage = C::kTileBytesA + C::kTileBytesB;
  auto ldsA = [&](int buf) { return lds + buf * kStage; };
  auto ldsB = [&](int buf) { return lds + buf * kStage + C::kTileBytesA; };

  // global -> LDS staging: thread covers chunk tid%8 of rows tid/8 + 32*i
  const int ld_row = tid >> 3;
  const int ld_chunk = tid & 7;
  u32x4 ra[C::kLoadsA], rb[C::kLoadsB];

  auto load_tiles = [&](int64_t kb) {
#pragma unroll
    for (int i = 0; i < C::kLoadsA; ++i) {
      const int r = ld_row + 32 * i;
      ra[i] = *reinterpret_cast<const u32x4*>(b + (n0 + r) * ld_b + kb * 128 + ld_chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < C::kLoadsB; ++i) {
      const int r = ld_row + 32 * i;
      const int64_t m = m0 + r;
      rb[i] = (m < m_end) ? *reinterpret_cast<const u32x4*>(a + m * ld_a + kb * 128 + ld_chunk * 16)
                          : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::kLoadsA; ++i)
      *reinterpret_cast<u32x4*>(ldsA(buf) + swz(ld_row + 32 * i, ld_chunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < C::kLoadsB; ++i)
      *reinterpret_cast<u32x4*>(ldsB(buf) + swz(ld_row + 32 * i, ld_chunk)) = rb[i];
  };

  // activation scale rows of this lane: m = m0 + wm + 16*j + lane%16
  float sa_next[WM];
  auto load_scales = [&](int64_t kb) {
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int64_t m = m0 + wm + 16 * j + (lane & 15);
      sa_next[j] = (m < m_end) ? as[kb * ld_as + m] : 0.0f;
    }
  };

  v4f acc[WN][WM];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int64_t nb = n0 / 128;
  const int frag_row = lane & 15;
  const int frag_chunk = (lane >> 4) * 2;  // 32 bytes = chunks 2q, 2q+1

  load_tiles(0);
  load_scales(0);
  store_tiles(0);
  __syncthreads();

  for (int64_t kb = 0; kb < kblocks; ++kb) {
    const int buf = kb & 1;
    float sa[WM];
#pragma unroll
    for (int j = 0; j < WM; ++j) sa[j] = sa_next[j];
    const float sb = bs[nb * kblocks + kb];
    if (kb + 1 < kblocks) {
      load_tiles(kb + 1);
      load_scales(kb + 1);
    }
    // B fragments (activations) for this wave's m tiles
    v8i fb[WM];
#pragma unroll
    for (int j = 0; j < WM; ++j) {
      const int r = wm + 16 * j + frag_row;
      u32x4 lo = *reinterpret_cast<const u32x4*>(ldsB(buf) + swz(r, frag_chunk));
      u32x4 hi = *reinterpret_cast<const u32x4*>(ldsB(buf) + swz(r, frag_chunk + 1));
      fb[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    float sab[WM];
#pragma unroll
    for (int j = 0; j < WM; ++j) sab[j] = sa[j] * sb;
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int r = wn + 16 * i + frag_row;
      u32x4 lo = *reinterpret_cast<const u32x4*>(ldsA(buf) + swz(r, frag_chunk));
      u32x4 hi = *reinterpret_cast<const u32x4*>(ldsA(buf) + swz(r, frag_chunk + 1));
      v8i fa = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        v4f p = mfma_fp8(fa, fb[j]);
        acc[i][j] = p * sab[j] + acc[i][j];
      }
    }
    if (kb + 1 < kblocks) {
      store_tiles(buf ^ 1);
    }
    __syncthreads();
  }

  // epilogue: lane holds y[m][n .. n+3], m = m0 + wm + 16j + lane%16, n = n0 + wn + 16i + 4*(lane/16)
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int64_t m = m0 + wm + 16 * j + (lane & 15);
    if (m >= m_end) continue;
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const int64_t n = n0 + wn + 16 * i + 4 * (lane >> 4);
      uint2 o;
      o.x = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
      o.y = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
      *reinterpret_cast<uint2*>(y + m * ld_y + n) = o;
    }
  }
}

constexpr int kWN = 4, kWM = 4;
using DenseCfg = TileCfg<kWN, kWM>;
constexpr int kLdsBytes = 2 * (DenseCfg::kTileBytesA + DenseCfg::kTileBytesB);

__global__ __launch_bounds__(256) void gemm_w8a8_kernel(const uint8_t* __restrict__ a, int64_t ld_a,
                                                        const float* __restrict__ as, int64_t ld_as,
                                                        const uint8_t* __restrict__ b, int64_t ld_b,
                                                        const float* __restrict__ bs, uint16_t* __restrict__ y,
                                                        int64_t ld_y, int64_t m, int64_t n, int64_t kblocks,
                                                        int n_tiles) {
  __shared__ __align__(16) uint8_t lds[kLdsBytes];
  const int64_t tile_n = blockIdx.x % n_tiles;
  const int64_t tile_m = blockIdx.x / n_tiles;
  gemm_tile<kWN, kWM>(a, ld_a, as, ld_as, b, ld_b, bs, y, ld_y, tile_m * DenseCfg::BM, m,
                      tile_n * DenseCfg::BN, kblocks, lds);
}

hipError_t launch_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                       int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
  const int n_tiles = (int)(n / DenseCfg::BN);
  const int64_t m_tiles = (m + DenseCfg::BM - 1) / DenseCfg::BM;
  hipLaunchKernelGGL(gemm_w8a8_kernel, dim3((unsigned)(n_tiles * m_tiles)), dim3(256), 0, stream,
                     reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as,
                     reinterpret_cast<const uint8_t*>(b), ld_b, b_s, reinterpret_cast<uint16_t*>(y), ld_y,
                     m, n, k / 128, n_tiles);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Grouped: rows of `a` are sorted by expert; rows [off[g], off[g+1]) use b[g].
// The tile schedule is derived on the device from the offsets: the grid is sized
// for the worst case (ceil(total_m / BM) + G m-tiles); each workgroup counts the
// m-tiles of the groups before it to find its (group, m-tile) and exits if it has
// none.  No host synchronization, no workspace.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(256) void grouped_gemm_w8a8_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, const float* __restrict__ bs, const int32_t* __restrict__ off,
    int32_t groups, uint16_t* __restrict__ y, int64_t ld_y, int64_t n, int64_t k, int n_tiles) {
  __shared__ __align__(16) uint8_t lds[kLdsBytes];
  __shared__ int32_t sel[2];
  const int64_t tile_n = blockIdx.x % n_tiles;
  const int64_t tile_m = blockIdx.x / n_tiles;  // global m-tile index
  if (threadIdx.x < 64) {
    // prefix over groups of ceil(rows / BM), 64 groups per pass
    const int lane = threadIdx.x;
    int64_t base = 0;
    int found_g = -1;
    int64_t found_t = 0;
    for (int g0 = 0; g0 < groups && found_g < 0; g0 += 64) {
      const int g = g0 + lane;
      int64_t tiles = 0;
      if (g < groups) tiles = (off[g + 1] - off[g] + DenseCfg::BM - 1) / DenseCfg::BM;
      // inclusive scan across the wave
      int64_t incl = tiles;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int64_t o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
      }
      const int64_t excl = incl - tiles;
      const bool mine = (g < groups) && (tile_m >= base + excl) && (tile_m < base + incl);
      const unsigned long long hit = __ballot(mine);
      if (hit) {
        const int src = __ffsll(hit) - 1;
        found_g = g0 + src;
        found_t = tile_m - base - __shfl(excl, src);
      }
      base += __shfl(incl, 63);
    }
    if (lane == 0) {
      sel[0] = found_g;
      sel[1] = (int32_t)found_t;
    }
  }
  __syncthreads();
  const int g = sel[0];
  if (g < 0) return;
  const int64_t kblocks = k / 128;
  const int64_t row0 = off[g] + (int64_t)sel[1] * DenseCfg::BM;
  gemm_tile<kWN, kWM>(a, ld_a, as, ld_as, b + (int64_t)g * n * k, k, bs + (int64_t)g * (n / 128) * kblocks,
                      y, ld_y, row0, off[g + 1], tile_n * DenseCfg::BN, kblocks, lds);
}

hipError_t launch_grouped_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                               const void* b, const float* b_s, const int32_t* offsets, int32_t groups,
                               int64_t total_m, void* y, int64_t ld_y, int64_t n, int64_t k,
                               hipStream_t stream) {
  const int n_tiles = (int)(n / DenseCfg::BN);
  const int64_t m_tiles = (total_m + DenseCfg::BM - 1) / DenseCfg::BM + groups;
  hipLaunchKernelGGL(grouped_gemm_w8a8_kernel, dim3((unsigned)(n_tiles * m_tiles)), dim3(256), 0,
                     stream, reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as,
                     reinterpret_cast<const uint8_t*>(b), b_s, offsets, groups,
                     reinterpret_cast<uint16_t*>(y), ld_y, n, k, n_tiles);
  return hipGetLastError();
}

}  // namespace fp8q

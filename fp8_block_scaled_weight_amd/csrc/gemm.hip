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
// Matrix core.  Each 128-wide K block is exactly one v_mfma_f32_16x16x128_f8f6f4 per
// 16x16 output tile, started from a zero accumulator, so P_kb leaves the matrix core
// whole and is folded into the running fp32 sum with one FMA per element.  The MFMA's
// A operand is 16 weight rows (n) and its B operand 16 token rows (m); both are
// K-contiguous and loaded the same way (lane l: row l%16, bytes 32*(l/16)..+31 of the
// 128-byte K block), so whatever K order the matrix core uses applies to both.  The
// result gives lane l the outputs m = l%16, n = 4*(l/16) + r (r < 4): one token scale
// per lane and tile, four consecutive outputs per store.
//
// Data movement.  A workgroup owns a BM x BN output tile and walks K in 128-byte steps.
// Each step's operand rows (BN weight rows, then BM token rows, 128 bytes each) are
// copied HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging) into a ring of
// STAGES buffers, STAGES-1 steps ahead of the step being multiplied.  In LDS the
// 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7): the copies write 1 KB
// (8 rows) per wave instruction in lane order, so each lane fetches the chunk that
// belongs at its slot.  Fragments are read 8 bytes at a time (ds_read_b64, four per
// lane and fragment): such a read is served a half-wave (32 lanes) at a time across
// the 64 four-byte banks, the swizzle gives the 16 rows of a fragment 16 distinct
// (row parity, chunk) bank groups, and lanes of odd 16-lane groups take the two
// halves of each chunk in the opposite order, so every half-wave touches each bank
// once (16-byte reads of the same data conflict two ways: the LDS bank-conflict
// counter shows the difference).  The half swap permutes the K bytes of those lanes
// identically for both operands, so the matrix core still pairs a[m][k] with b[n][k].
// Reads carry explicit waits tied to their registers, and each step is entered
// through one "wait for my copies, then barrier" sequence, so copies for later steps
// stay in flight across the multiply.
#include <utility>

#include "launch.hpp"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define FP8Q_GLOBAL __attribute__((address_space(1)))
#define FP8Q_LDS __attribute__((address_space(3)))

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

template <int IMM>
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(IMM));
  return v;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int IMM>
__device__ __forceinline__ u32x2 lds_read8(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(IMM));
  return v;
}

// One MFMA operand fragment (32 bytes per lane) as four 8-byte reads: chunk pair
// (lo, hi), halves in the order hsw, hsw ^ 8 (hsw = 8 on odd 16-lane groups).
constexpr int kReadsPerFragment = 4;

template <int IMM>
__device__ __forceinline__ v8i read_fragment(uint32_t lo, uint32_t hi, uint32_t hsw) {
  const u32x2 p0 = lds_read8<IMM>(lo + hsw), p1 = lds_read8<IMM>(lo + (hsw ^ 8));
  const u32x2 p2 = lds_read8<IMM>(hi + hsw), p3 = lds_read8<IMM>(hi + (hsw ^ 8));
  return v8i{(int)p0.x, (int)p0.y, (int)p1.x, (int)p1.y, (int)p2.x, (int)p2.y, (int)p3.x, (int)p3.y};
}

// Wait until at most N LDS reads are outstanding; ties the wait to x so that no use of
// x can be scheduled before it.
template <int N>
__device__ __forceinline__ void lds_wait(v8i& x) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}

__device__ __forceinline__ v8i join(u32x4 lo, u32x4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WAVES_M / 16;  // 16x16 tiles per wave along m (tokens)
  static constexpr int WN = BN / WAVES_N / 16;  // along n (weights)
  static constexpr int ROWS = BN + BM;          // rows staged per K step: weights, then tokens
  static constexpr int A_BYTES = BN * 128;      // weight rows of a stage
  static constexpr int SCALE_OFF = ROWS * 128;  // token scales of a stage (BM floats)
  static constexpr int STAGE_BYTES = ((ROWS * 128 + BM * 4) + 1023) / 1024 * 1024;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int LOADS = ROWS / (8 * WAVES);    // 16-byte operand copies per thread per step
  static constexpr int LOADS_W = BN / (8 * WAVES);    // of which weight rows
  static constexpr int SCALES_PER_WAVE = BM / WAVES;  // 4-byte token-scale copies per wave per step
  static_assert(ROWS % (8 * WAVES) == 0 && BN % (8 * WAVES) == 0, "whole 1 KB copies per wave");
  static_assert(BN / WAVES_N <= 128 && 128 % (BN / WAVES_N) == 0, "a wave's n range is one scale block");
  static_assert(SCALES_PER_WAVE <= 64 && BM % WAVES == 0, "one scale copy per wave");
  static_assert(WM % 4 == 0, "a lane's token scales are read 4 at a time");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && WM >= 1 && WN >= 1 && WM % 2 == 0, "");
  static_assert((STAGES - 2) * (LOADS + 1) <= 63, "vmcnt range");
};

constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit dwords (gfx9 layout)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcFlags);
}

// Keep uses of x after the preceding wait (no code is emitted).
template <class T>
__device__ __forceinline__ void after_wait(T& x) {
  asm volatile("" : "+v"(x));
}

// LDS placement of 16-byte chunk c of staged row r: chunk c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// One BM x BN output tile: token rows [m0, m_end) (m_end - m0 may be < BM), weight
// rows [n0, n0 + BN).  b / bs describe this tile's weight matrix and its scales.
// a_rows and b_rows bound the operand buffers (rows, row pitch ld_a / ld_b bytes).
template <class C>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ a, int64_t ld_a, int64_t a_rows,
                                          const float* __restrict__ as, int64_t ld_as,
                                          const uint8_t* __restrict__ b, int64_t ld_b,
                                          const float* __restrict__ bs, int kblocks,
                                          uint16_t* __restrict__ y, int64_t ld_y, int64_t m0, int64_t m_end,
                                          int64_t n0, uint8_t FP8Q_LDS* lds) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer-resource builtins exist in the device pass only
  constexpr int S = C::STAGES;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave / C::WAVES_N) * C::WM * 16;
  const int wn = (wave % C::WAVES_N) * C::WN * 16;

  // ---- copy sources: lane byte offsets that stay fixed while K advances (token rows
  // past m_end are clamped to the last row: valid memory, never stored)
  uint32_t src[C::LOADS];
  {
    const int r_in = lane >> 3;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int r = (i * C::WAVES + wave) * 8 + r_in;
      const int chunk = (lane & 7) ^ swz(r);
      if (i < C::LOADS_W) {
        src[i] = (uint32_t)((n0 + r) * ld_b) + chunk * 16;
      } else {
        int64_t m = m0 + (r - C::BN);
        m = m < m_end ? m : m_end - 1;
        src[i] = (uint32_t)(m * ld_a) + chunk * 16;
      }
    }
  }
  // token-scale copy: lane i of wave w fills scale slot p = w*SCALES_PER_WAVE + i.  A
  // wave's token rows wm + 16j + r (j < WM, r < 16) sit at slots wm + r*WM + j, so the
  // WM scales a lane needs are contiguous and come in with 16-byte reads (which, unlike
  // broadcast 4-byte reads, cost no bank-conflict cycles).
  const int slot = wave * C::SCALES_PER_WAVE + lane;
  const int slab = slot / (16 * C::WM), within = slot % (16 * C::WM);
  int64_t srow = m0 + slab * 16 * C::WM + (within % C::WM) * 16 + within / C::WM;
  srow = srow < m_end ? srow : m_end - 1;
  const uint32_t ssrc = (uint32_t)(srow * 4);
  const bool scale_lane = lane < C::SCALES_PER_WAVE;

  const uint32_t a_bytes = (uint32_t)(a_rows * ld_a);
  const uint32_t b_bytes = (uint32_t)((n0 + C::BN) * ld_b);
  auto issue = [&](int kb) {
    uint8_t FP8Q_LDS* dst = lds + (kb % S) * C::STAGE_BYTES;
    const __amdgpu_buffer_rsrc_t rb = rsrc(b + (size_t)kb * 128, b_bytes - kb * 128);
    const __amdgpu_buffer_rsrc_t ra = rsrc(a + (size_t)kb * 128, a_bytes - kb * 128);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(i < C::LOADS_W ? rb : ra,
                                               (FP8Q_LDS void*)(dst + (i * C::WAVES + wave) * 1024), 16, src[i], 0, 0,
                                               0);
    const __amdgpu_buffer_rsrc_t rs = rsrc(as + (size_t)kb * ld_as, (uint32_t)(ld_as * 4));
    if (scale_lane)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FP8Q_LDS void*)(dst + C::SCALE_OFF + wave * C::SCALES_PER_WAVE * 4),
                                               4, ssrc, 0, 0, 0);
  };

  // ---- fragment read addresses (lane part; stage and tile offsets added per step)
  const int x = swz(lane & 15);  // fragment rows start at multiples of 16
  const int q2 = (lane >> 4) * 2;
  const uint32_t rd_lo = (lane & 15) * 128 + ((q2 ^ x) << 4);
  const uint32_t rd_hi = (lane & 15) * 128 + (((q2 + 1) ^ x) << 4);
  const uint32_t hsw = ((lane >> 4) & 1) * 8;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const int64_t sb_base = ((n0 + wn) / 128) * kblocks;

  v4f acc[C::WN][C::WM];
#pragma unroll
  for (int i = 0; i < C::WN; ++i)
#pragma unroll
    for (int j = 0; j < C::WM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // prologue: copies for steps 0 .. S-2
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < kblocks) issue(s);
  float sb_next = bs[sb_base];

  for (int kb = 0; kb < kblocks; ++kb) {
    const float sb = sb_next;
    if (kb + 1 < kblocks) sb_next = bs[sb_base + kb + 1];

    // Wait until this thread's copies for step kb have landed (the copies of up to S-2
    // later steps may stay in flight), then barrier: after it every thread's copies for
    // kb are in LDS and no wave still reads the buffer of step kb-1, which the copy
    // issued next reuses.
    if (kb + S - 2 < kblocks) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((S - 2) * (C::LOADS + 1)) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (kb + S - 1 < kblocks) issue(kb + S - 1);

    const uint32_t stage = lds_base + (uint32_t)((kb % S) * C::STAGE_BYTES);
    const uint32_t a_lo = stage + wn * 128 + rd_lo, a_hi = stage + wn * 128 + rd_hi;
    const uint32_t b_lo = stage + C::A_BYTES + wm * 128 + rd_lo, b_hi = stage + C::A_BYTES + wm * 128 + rd_hi;
    const uint32_t s_addr = stage + C::SCALE_OFF + (wm + (lane & 15) * C::WM) * 4;

    v8i fa[C::WN];
    v8i fb[3];
    u32x4 sq[C::WM / 4];
    // weight fragments of all n tiles, token scales, token fragment 0
    [&]<int... I>(std::integer_sequence<int, I...>) {
      ((fa[I] = read_fragment<I * 2048>(a_lo, a_hi, hsw)), ...);
    }(std::make_integer_sequence<int, C::WN>{});
    [&]<int... P>(std::integer_sequence<int, P...>) {
      ((sq[P] = lds_read16<16 * P>(s_addr)), ...);
    }(std::make_integer_sequence<int, C::WM / 4>{});
    fb[0] = read_fragment<0>(b_lo, b_hi, hsw);

    // token tile j: prefetch fragment j+1 (3 rotating registers keep a fragment's
    // registers untouched until well after the MFMAs that read them), wait for j,
    // then one MFMA per weight tile and its promotion FMA
    [&]<int... J>(std::integer_sequence<int, J...>) {
      (
          [&] {
            constexpr int j = J;
            if constexpr (j + 1 < C::WM) {
              fb[(j + 1) % 3] = read_fragment<(j + 1) * 2048>(b_lo, b_hi, hsw);
              lds_wait<kReadsPerFragment>(fb[j % 3]);
            } else {
              lds_wait<0>(fb[j % 3]);
            }
            if constexpr (j == 0) {
#pragma unroll
              for (int i = 0; i < C::WN; ++i) after_wait(fa[i]);
#pragma unroll
              for (int jj = 0; jj < C::WM / 4; ++jj) after_wait(sq[jj]);
            }
            const float sab = __uint_as_float(sq[j / 4][j % 4]) * sb;
#pragma unroll
            for (int i = 0; i < C::WN; ++i) {
              v4f p = mfma_fp8(fa[i], fb[j % 3]);
              acc[i][j] = p * sab + acc[i][j];
            }
          }(),
          ...);
    }(std::make_integer_sequence<int, C::WM>{});
  }

  // ---- epilogue: lane holds y[m][n .. n+3], m = m0 + wm + 16j + lane%16,
  // n = n0 + wn + 16i + 4*(lane/16); one bf16 rounding per output
#pragma unroll
  for (int j = 0; j < C::WM; ++j) {
    const int64_t m = m0 + wm + 16 * j + (lane & 15);
    if (m >= m_end) continue;
#pragma unroll
    for (int i = 0; i < C::WN; ++i) {
      const int64_t n = n0 + wn + 16 * i + 4 * (lane >> 4);
      uint2 o;
      o.x = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
      o.y = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
      *reinterpret_cast<uint2*>(y + m * ld_y + n) = o;
    }
  }
#endif
}

// Tile order.  Workgroups are dealt to the 8 XCDs round-robin, so consecutive tile
// indices are given to one XCD: its L2 then serves a compact block of tiles
// (GROUP_M token tiles x all weight tiles, walked weight-tile-major) that share
// operand rows.
constexpr int kXcds = 8;

__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t tiles) {
  const int64_t per = (tiles + kXcds - 1) / kXcds;
  return (bid % kXcds) * per + bid / kXcds;
}

template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int64_t t, int64_t m_tiles, int64_t n_tiles, int64_t& tm, int64_t& tn) {
  const int64_t span = (int64_t)GROUP_M * n_tiles;
  const int64_t grp = t / span;
  const int64_t first = grp * GROUP_M;
  const int64_t gm = (m_tiles - first) < GROUP_M ? (m_tiles - first) : GROUP_M;
  const int64_t r = t - grp * span;
  tm = first + r % gm;
  tn = r / gm;
}

// Two waves per SIMD (8 per workgroup): while one wave waits for LDS or a barrier, the
// other keeps the matrix core busy, and one wave's promotion FMAs overlap the other's
// MFMAs.
using CfgLarge = GemmCfg<256, 256, 2, 4, 2>;   // 128 x 64 per wave, 130 KB LDS
using CfgMid = GemmCfg<128, 128, 2, 4, 2>;     // 64 x 32 per wave, 66 KB LDS
using CfgSmall = GemmCfg<128, 64, 2, 2, 4>;    // 64 x 32 per wave, 4 waves: more tiles for mid-size M

template <class C>
__global__ __launch_bounds__(C::THREADS) void gemm_w8a8_kernel(const uint8_t* __restrict__ a, int64_t ld_a,
                                                                const float* __restrict__ as, int64_t ld_as,
                                                                const uint8_t* __restrict__ b, int64_t ld_b,
                                                                const float* __restrict__ bs,
                                                                uint16_t* __restrict__ y, int64_t ld_y, int64_t m,
                                                                int64_t m_tiles, int64_t n_tiles, int kblocks) {
  __shared__ __align__(1024) uint8_t lds[C::LDS_BYTES];
  const int64_t tiles = m_tiles * n_tiles;
  const int64_t t = xcd_tile(blockIdx.x, tiles);
  if (t >= tiles) return;
  int64_t tm, tn;
  tile_coords<4>(t, m_tiles, n_tiles, tm, tn);
  const int64_t m0 = tm * C::BM;
  const int64_t m_end = (m0 + C::BM) < m ? (m0 + C::BM) : m;
  gemm_tile<C>(a, ld_a, m, as, ld_as, b, ld_b, bs, kblocks, y, ld_y, m0, m_end, tn * C::BN,
               (uint8_t FP8Q_LDS*)lds);
}

template <class C>
static hipError_t launch_dense(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                               int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                               int64_t k, hipStream_t stream) {
  const int64_t n_tiles = n / C::BN;
  const int64_t m_tiles = (m + C::BM - 1) / C::BM;
  const int64_t tiles = m_tiles * n_tiles;
  const int64_t grid = ((tiles + kXcds - 1) / kXcds) * kXcds;
  hipLaunchKernelGGL(gemm_w8a8_kernel<C>, dim3((unsigned)grid), dim3(C::THREADS), 0, stream,
                     reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b),
                     ld_b, b_s, reinterpret_cast<uint16_t*>(y), ld_y, m, m_tiles, n_tiles, (int)(k / 128));
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Few tokens (decode, short prefill): the GEMM streams the weight matrix once and is
// HBM-bound, so it is spread over as many CUs as possible.  A workgroup owns 16 weight
// rows and up to 16*WM token rows; its 8 waves take the K blocks round-robin and load
// their fragments straight into registers (weights read once, with a non-temporal
// hint; token rows come from L2).  The 8 partial sums are added through LDS in a fixed
// order, so the result does not depend on timing.
// ----------------------------------------------------------------------------
constexpr int kSmallWaves = 8;

template <int WM>
__global__ __launch_bounds__(64 * kSmallWaves) void gemm_smallm_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, int64_t ld_b, const float* __restrict__ bs, uint16_t* __restrict__ y,
    int64_t ld_y, int64_t m, int64_t n16, int kblocks) {
  __shared__ v4f part[kSmallWaves][WM][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tn = blockIdx.x % n16;
  const int64_t m0 = (blockIdx.x / n16) * (16 * WM);
  const int64_t n0 = tn * 16;
  const int q = lane >> 4;
  const uint8_t* brow = b + (n0 + (lane & 15)) * ld_b + q * 32;
  const uint8_t* arow[WM];
  int64_t srow[WM];  // token row of this lane (row 0 stands in for rows past m)
  bool live[WM];
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int64_t r = m0 + 16 * j + (lane & 15);
    live[j] = r < m;
    srow[j] = live[j] ? r : 0;
    arow[j] = a + srow[j] * ld_a + q * 32;
  }
  const float* bsrow = bs + (n0 / 128) * kblocks;
  v4f acc[WM];
#pragma unroll
  for (int j = 0; j < WM; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  constexpr int U = WM >= 4 ? 2 : 4;  // K blocks in flight per wave (register budget permitting)
  for (int kb0 = wave; kb0 < kblocks; kb0 += kSmallWaves * U) {
    v8i fw[U], ft[U][WM];
    float sa[U][WM], sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u * kSmallWaves;
      if (kb < kblocks) {
        const u32x4* pw = reinterpret_cast<const u32x4*>(brow + (int64_t)kb * 128);
        fw[u] = join(__builtin_nontemporal_load(pw), __builtin_nontemporal_load(pw + 1));
        sb[u] = bsrow[kb];
#pragma unroll
        for (int j = 0; j < WM; ++j) {
          const u32x4* pt = reinterpret_cast<const u32x4*>(arow[j] + (int64_t)kb * 128);
          ft[u][j] = live[j] ? join(pt[0], pt[1]) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
          const float sv = as[(int64_t)kb * ld_as + srow[j]];
          sa[u][j] = live[j] ? sv : 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u * kSmallWaves;
      if (kb < kblocks) {
#pragma unroll
        for (int j = 0; j < WM; ++j) {
          v4f p = mfma_fp8(fw[u], ft[u][j]);
          acc[j] = p * (sa[u][j] * sb[u]) + acc[j];
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < WM; ++j) part[wave][j][lane] = acc[j];
  __syncthreads();
  // wave j < WM adds the 8 partial sums of token tile j (fixed order) and stores it
  if (wave < WM) {
    const int j = wave;
    v4f t = part[0][j][lane];
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w) t += part[w][j][lane];
    const int64_t row = m0 + 16 * j + (lane & 15);
    if (row < m) {
      const int64_t col = n0 + 4 * q;
      uint2 o;
      o.x = bf16_rne(t[0]) | (bf16_rne(t[1]) << 16);
      o.y = bf16_rne(t[2]) | (bf16_rne(t[3]) << 16);
      *reinterpret_cast<uint2*>(y + row * ld_y + col) = o;
    }
  }
}

template <int WM>
static hipError_t launch_smallm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                                int64_t k, hipStream_t stream) {
  const int64_t n16 = n / 16;
  const int64_t groups = (m + 16 * WM - 1) / (16 * WM);
  hipLaunchKernelGGL(gemm_smallm_kernel<WM>, dim3((unsigned)(n16 * groups)), dim3(64 * kSmallWaves), 0, stream,
                     reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b), ld_b,
                     b_s, reinterpret_cast<uint16_t*>(y), ld_y, m, n16, (int)(k / 128));
  return hipGetLastError();
}

hipError_t launch_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                       int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
  // few tokens: stream the weights over all CUs
  if (m <= 16) return launch_smallm<1>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  if (m <= 32) return launch_smallm<2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  if (m <= 64) return launch_smallm<4>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  if (m < 1024) return launch_dense<CfgSmall>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  // large tiles when they still give every CU a tile
  const int64_t large_tiles = ((m + CfgLarge::BM - 1) / CfgLarge::BM) * (n / CfgLarge::BN);
  if (large_tiles >= 256)
    return launch_dense<CfgLarge>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  return launch_dense<CfgMid>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
}

// ----------------------------------------------------------------------------
// Grouped: rows of `a` are sorted by expert; rows [off[g], off[g+1]) use b[g].
// The tile schedule is derived on the device from the offsets: the grid is sized
// for the worst case (ceil(total_m / BM) + G m-tiles); each workgroup counts the
// m-tiles of the groups before it to find its (group, m-tile) and exits if it has
// none.  No host synchronization, no workspace.
// ----------------------------------------------------------------------------
using CfgGrouped = CfgMid;

template <class C>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_w8a8_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, const float* __restrict__ bs, const int32_t* __restrict__ off,
    int32_t groups, uint16_t* __restrict__ y, int64_t ld_y, int64_t n, int64_t k, int64_t n_tiles) {
  __shared__ __align__(1024) uint8_t lds[C::LDS_BYTES];
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
      if (g < groups) tiles = (off[g + 1] - off[g] + C::BM - 1) / C::BM;
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
  const int kblocks = (int)(k / 128);
  const int64_t row0 = off[g] + (int64_t)sel[1] * C::BM;
  const int64_t row_end = (row0 + C::BM) < off[g + 1] ? (row0 + C::BM) : off[g + 1];
  const int64_t a_rows = off[groups];
  const uint8_t* bg = b + (int64_t)g * n * k;
  const float* bsg = bs + (int64_t)g * (n / 128) * kblocks;
  gemm_tile<C>(a, ld_a, a_rows, as, ld_as, bg, k, bsg, kblocks, y, ld_y, row0, row_end, tile_n * C::BN,
               (uint8_t FP8Q_LDS*)lds);
}

hipError_t launch_grouped_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                               const void* b, const float* b_s, const int32_t* offsets, int32_t groups,
                               int64_t total_m, void* y, int64_t ld_y, int64_t n, int64_t k,
                               hipStream_t stream) {
  using C = CfgGrouped;
  const int64_t n_tiles = n / C::BN;
  const int64_t m_tiles = (total_m + C::BM - 1) / C::BM + groups;
  hipLaunchKernelGGL(grouped_gemm_w8a8_kernel<C>, dim3((unsigned)(n_tiles * m_tiles)), dim3(C::THREADS), 0, stream,
                     reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b), b_s,
                     offsets, groups, reinterpret_cast<uint16_t*>(y), ld_y, n, k, n_tiles);
  return hipGetLastError();
}

}  // namespace fp8q

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
// Matrix core.  A 128-wide K block of a 32x32 output tile is two chained
// v_mfma_f32_32x32x64_f8f6f4 (K halves 0 and 1) started from a zero accumulator, so
// P_kb leaves the matrix core whole and is folded into the running fp32 sum with one
// FMA per element.  The MFMA's A operand is 32 weight rows (n) and its B operand 32
// token rows (m); both are K-contiguous and loaded the same way (lane l: row l%32,
// bytes 32*(l/32)..+31 of the K half), so whatever K order the matrix core uses applies
// to both.  The result gives lane l the token m = l%32 and the weights
// n = 8q + 4*(l/32) + r (q, r < 4): one token scale per lane and tile.
//
// Data movement.  A workgroup owns a BM x BN output tile and walks K in 128-byte steps.
// Each step's operand rows (BN weight rows, then BM token rows, 128 bytes each) and
// its scales are copied HBM -> LDS with buffer loads that write LDS directly (no VGPR
// staging) into a ring of STAGES buffers, STAGES-1 steps ahead of the step being
// multiplied.  In LDS the 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7):
// the copies write 1 KB (8 rows) per wave instruction in lane order, so each lane
// fetches the chunk that belongs at its slot; a 16-byte fragment read then gives the
// 16 lanes served together 16 distinct (row parity, chunk) bank groups.  The copies
// are issued in inline asm so that the compiler, which does not see them, schedules
// and counts the LDS fragment reads on its own; each step is entered through one
// "wait for my copies, then barrier" sequence, so copies for later steps stay in
// flight across the multiply.
#include <utility>

#include "e4m3.hpp"
#include "launch.hpp"
#include "swiglu.hpp"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define FP8Q_LDS __attribute__((address_space(3)))

// 16x16x128 FP8 MFMA from a zero accumulator (scale operands 0 select the unscaled
// FP8 x FP8 -> fp32 instruction)
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8i join(u32x4 lo, u32x4 hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// 32x32x64 FP8 MFMA accumulating into c (unscaled form, as above)
__device__ __forceinline__ v16f mfma32(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same with block scales applied by the matrix core: lane l passes the E8M0
// exponent (bias 127) of row l%32 of the A operand and of column l%32 of the B operand
// for the 32-wide K group the lane's data belong to.  A power-of-two binary32 scale
// 2^e (e >= -127) has E8M0 code bits >> 23.
__device__ __forceinline__ v16f mfma32_scaled(v8i a, v8i b, v16f c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}
__device__ __forceinline__ int e8m0_of(float pow2_scale) { return (int)(__float_as_uint(pow2_scale) >> 23); }

// KSPLIT > 1: the workgroup holds KSPLIT groups of WAVES_M x WAVES_N waves.  Group g takes
// the K blocks g, g + KSPLIT, ... through its own copy ring, in lockstep with the others
// (one barrier per step for all), and at the end the groups' partial sums are added in
// group order through LDS.  It doubles the waves per SIMD of a small tile without a
// workspace.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int KSPLIT_ = 1>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, STAGES = STAGES_;
  static constexpr int KSPLIT = KSPLIT_;
  static constexpr int GW = WAVES_M * WAVES_N;                // waves per K group
  static constexpr int WAVES = GW * KSPLIT;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // wave tile: tokens x weights
  static constexpr int JM = TM / 32, IN = TN / 32;            // 32x32 sub-tiles per wave
  static constexpr int ROWS = BN + BM;                        // staged rows: weights, then tokens
  static constexpr int SCALE_OFF = ROWS * 128;
  static constexpr int SPW = BM / GW;                         // token scales copied per wave
  static constexpr int NWS = BN >= 128 ? BN / 128 : 1;        // weight scales per step
  static constexpr int WSC_OFF = SCALE_OFF + BM * 4;            // per-wave weight scales
  static constexpr int STAGE_BYTES = ((WSC_OFF + GW * NWS * 4) + 1023) / 1024 * 1024;
  static constexpr int LDS_BYTES = KSPLIT * STAGES * STAGE_BYTES;
  static constexpr int LOADS = ROWS / (8 * GW);
  static constexpr int LOADS_W = BN / (8 * GW);
  static constexpr int VM_PER_STEP = LOADS + 2;  // copies per thread and step
  static constexpr int RED_OFF = BM * BN * 2;    // KSPLIT > 1: partial sums, after the epilogue stage
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32x32 sub-tiles");
  static_assert(ROWS % (8 * GW) == 0 && BN % (8 * GW) == 0, "whole 1 KB copies per wave");
  static_assert(TN <= 128 && 128 % TN == 0, "a wave's weight rows lie in one scale block");
  static_assert(SPW >= 1 && SPW + NWS <= 64 && BM % GW == 0, "scale copies");
  static_assert(JM == 2 || JM == 4, "token scales per lane; the deferred chain's token "
                "fragment must not be the one the next step reads first");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(KSPLIT == 1 || RED_OFF + (KSPLIT - 1) * BM * BN * 4 <= LDS_BYTES, "partial sums fit in LDS");
  static_assert(STAGES >= 2 && (STAGES - 2) * VM_PER_STEP <= 63, "vmcnt range");
};

// Copies global -> LDS: lane i's 16 (or 4) bytes at rsrc base + voff + soff land at LDS
// address m0 + 16i (4i).  Issued in asm so that the compiler's own wait counting for
// LDS reads is not tied to these copies; the s_nop covers the one wait state an M0
// write needs before an LDS-writing buffer load.
__device__ __forceinline__ void dma16(v4i rs, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma4(v4i rs, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rs), "s"(soff), "{m0}"(lds_addr) : "memory");
}
// Raw buffer resource (stride 0, 32-bit data format) over [base, base + bytes).
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  r.y = __builtin_amdgcn_readfirstlane((int)((uint32_t)(p >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

// LDS placement of 16-byte chunk c of staged row r: chunk c ^ swz(r).
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <class T>
__device__ __forceinline__ T lds_ld(const uint8_t FP8Q_LDS* base, uint32_t off) {
  return *reinterpret_cast<const T FP8Q_LDS*>(base + off);
}

// SW (MoE fc1 with SwiGLU fused): B holds [gate; up] rows, `half` each.  A 256-wide tile
// jt = n0 / 256 multiplies gate rows 128jt .. +127 (tile columns 0..127) and up rows
// half + 128jt .. +127 (columns 128..255), and its epilogue writes, instead of y, the
// SwiGLU of the bf16-rounded outputs quantized per 1x128 group: codes q[m][128jt + c],
// scale s[jt * ld_s + m].
struct SwigluOut {
  uint8_t* q = nullptr;
  int64_t ld_q = 0;
  float* s = nullptr;
  int64_t ld_s = 0;
  int64_t half = 0;
};

template <class C, bool POW2, bool SW = false>
__device__ __forceinline__ void gemm_tile(const uint8_t* __restrict__ a, int64_t ld_a, int64_t a_rows,
                                          const float* __restrict__ as, int64_t ld_as,
                                          const uint8_t* __restrict__ b, int64_t ld_b,
                                          const float* __restrict__ bs, int kblocks,
                                          uint16_t* __restrict__ y, int64_t ld_y, int64_t m0, int64_t m_end,
                                          int64_t n0, uint8_t FP8Q_LDS* lds, const SwigluOut sw = SwigluOut{},
                                          const int32_t* __restrict__ tok = nullptr) {
  static_assert(!SW || (C::BN == 256 && C::TN == 64 && C::WAVES_N == 4 && C::THREADS == 512 && C::BM % 64 == 0),
                "the fused SwiGLU epilogue assumes the 256x256 tile");
  static_assert(C::KSPLIT == 1 || (!SW && !POW2), "K groups: fp32-scale GEMM only");
  const int64_t jt = n0 / 256;  // SW: the tile's 128-row gate and up blocks
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave_all / C::GW;   // K group
  const int wave = wave_all % C::GW;  // wave within its K group
  const int wm = (wave / C::WAVES_N) * C::TM;
  const int wn = (wave % C::WAVES_N) * C::TN;
  uint8_t FP8Q_LDS* const lds0 = lds;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds + (uint32_t)(grp * C::STAGES * C::STAGE_BYTES);
  lds += grp * C::STAGES * C::STAGE_BYTES;  // this group's copy ring
  // step s of this group multiplies K block s * KSPLIT + grp (the last block again, with
  // a zero scale product, where that passes the end)
  const int nsteps = (kblocks + C::KSPLIT - 1) / C::KSPLIT;
  auto kblock = [&](int step) {
    const int kb = step * C::KSPLIT + grp;
    return kb < kblocks ? kb : kblocks - 1;
  };

  // ---- copy sources (fixed while K advances; K enters through the scalar offset)
  uint32_t src[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int r = (i * C::GW + wave) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(r);
    if (i < C::LOADS_W) {
      const int64_t wr = SW ? (r < 128 ? 128 * jt + r : sw.half + 128 * jt + (r - 128)) : n0 + r;
      src[i] = (uint32_t)(wr * ld_b) + chunk * 16;
    } else {
      int64_t m = m0 + (r - C::BN);
      m = m < m_end ? m : m_end - 1;
      if (tok) m = tok[m];  // the row's token (a holds the token rows)
      src[i] = (uint32_t)(m * ld_a) + chunk * 16;
    }
  }
  // token scales: slot p of the stage's scale area holds token
  // (p / TM) * TM + 32 * (p % TM % JM) + (p % TM / JM), so a lane's JM scales are contiguous
  const int slot = wave * C::SPW + lane;
  const int seg = slot / C::TM, q = slot % C::TM;
  int64_t srow = m0 + seg * C::TM + 32 * (q % C::JM) + q / C::JM;
  srow = srow < m_end ? srow : m_end - 1;
  if (tok) srow = tok[srow];
  const uint32_t ssrc = (uint32_t)(srow * 4);
  const bool tok_lane = lane < C::SPW;
  // weight scales: every wave copies the tile's NWS weight scales (lanes SPW ..
  // SPW+NWS-1) into its own slots, so that each wave issues the same number of copies
  const bool wsc_lane = lane >= C::SPW && lane < C::SPW + C::NWS;
  const int64_t wsrow = SW ? ((lane - C::SPW) == 0 ? jt : sw.half / 128 + jt) : (n0 / 128) + (lane - C::SPW);
  const uint32_t wsrc = (uint32_t)(wsrow * kblocks * 4);

  const v4i ra = make_rsrc(a, (uint32_t)(a_rows * ld_a));
  const v4i rb = make_rsrc(b, (uint32_t)((SW ? 2 * sw.half : n0 + C::BN) * ld_b));
  const v4i rsa = make_rsrc(as, (uint32_t)(ld_as * kblocks * 4));
  const v4i rsb = make_rsrc(bs, (uint32_t)((SW ? 2 * sw.half / 128 : n0 / 128 + C::NWS) * kblocks * 4));

  // copies [i0, i1) of this thread's 16-byte row copies for step kb into stage `stage`
  auto issue_rows = [&](int kb, int stage, int i0, int i1) {
    const uint32_t dst = lds_base + (uint32_t)(stage * C::STAGE_BYTES);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      if (i >= i0 && i < i1)
        dma16(i < C::LOADS_W ? rb : ra, src[i], (uint32_t)kb * 128u, dst + (uint32_t)((i * C::GW + wave) * 1024));
  };
  auto issue_scales = [&](int kb, int stage) {
    const uint32_t dst = lds_base + (uint32_t)(stage * C::STAGE_BYTES);
    const uint32_t sdst = dst + C::SCALE_OFF + (uint32_t)(wave * C::SPW * 4);
    if (tok_lane) dma4(rsa, ssrc, (uint32_t)(kb * ld_as * 4), sdst);
    if (wsc_lane) dma4(rsb, wsrc, (uint32_t)kb * 4u, dst + C::WSC_OFF + (uint32_t)((wave * C::NWS - C::SPW) * 4));
  };
  auto issue = [&](int kb, int stage) {
    issue_rows(kb, stage, 0, C::LOADS);
    issue_scales(kb, stage);
  };
  // With two stages the next step's row copies are spread over the step, PER of them
  // behind each of the first MFMA chains: issued all at once, they hold a wave at the
  // copy queue before its first MFMA (4096^3: 79 -> 68 us).  In the last step the rows
  // copied are the last block again, in range and into the stage no later step reads,
  // so that no branch separates the chains (one spills the accumulators); the final
  // waits cover these copies.  Deeper rings keep issuing a step's copies at once,
  // where such tail copies would be several steps' worth.
  constexpr bool SPREAD = C::STAGES == 2;
  constexpr int PER = 2;

  // ---- fragment offsets: lane l reads row l%32 of a 32-row tile, 16-byte chunks
  // 4h + 2(l/32) + e (e = 0, 1) for the MFMA of K half h
  const int r32 = lane & 31, g = lane >> 5;
  uint32_t fo[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 2; ++e) fo[h][e] = (uint32_t)(r32 * 128 + (((4 * h + 2 * g + e) ^ swz(r32)) << 4));
  const uint32_t so = (uint32_t)(C::SCALE_OFF + (wm + r32 * C::JM) * 4);
  const uint32_t wso = (uint32_t)(C::WSC_OFF + (wave * C::NWS + wn / 128) * 4);

  v16f acc[C::IN][C::JM];
#pragma unroll
  for (int i = 0; i < C::IN; ++i)
#pragma unroll
    for (int j = 0; j < C::JM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  if constexpr (POW2) {
    // Power-of-two scales: the matrix core applies them, so a K step is two chained
    // scaled MFMAs per 32x32 sub-tile accumulating straight into the running sum, with
    // no promotion.  Weight fragments are read at the step start, token fragments one
    // sub-tile ahead.
    constexpr int S = C::STAGES;
#pragma unroll
    for (int p = 0; p < S - 1; ++p)
      if (p < kblocks) issue(p, p);
    int cur = 0;
    for (int kb = 0; kb < kblocks; ++kb) {
      if (kb + S - 2 < kblocks) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((S - 2) * C::VM_PER_STEP) : "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
      const bool more = kb + S - 1 < kblocks;
      const int nst = cur == 0 ? S - 1 : cur - 1;
      const int kn = more ? kb + S - 1 : kblocks - 1;
      if constexpr (SPREAD) {
        if (more) issue_scales(kn, nst);
      } else {
        if (more) issue(kn, nst);
      }
      const uint8_t FP8Q_LDS* st = lds + cur * C::STAGE_BYTES;
      const uint8_t FP8Q_LDS* stw = st + wn * 128;
      const uint8_t FP8Q_LDS* stt = st + (C::BN + wm) * 128;
      v8i fa[C::IN][2];
#pragma unroll
      for (int i = 0; i < C::IN; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          fa[i][h] = join(lds_ld<u32x4>(stw, fo[h][0] + i * 4096), lds_ld<u32x4>(stw, fo[h][1] + i * 4096));
      int eb[C::JM];
      if constexpr (C::JM == 4) {
        const u32x4 t = lds_ld<u32x4>(st, so);
        eb[0] = (int)(t.x >> 23); eb[1] = (int)(t.y >> 23); eb[2] = (int)(t.z >> 23); eb[3] = (int)(t.w >> 23);
      } else {
        const u32x2 t = lds_ld<u32x2>(st, so);
        eb[0] = (int)(t.x >> 23); eb[1] = (int)(t.y >> 23);
      }
      const int ea = e8m0_of(lds_ld<float>(st, wso));
#pragma unroll
      for (int j = 0; j < C::JM; ++j) {
        v8i fb[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          fb[h] = join(lds_ld<u32x4>(stt, fo[h][0] + j * 4096), lds_ld<u32x4>(stt, fo[h][1] + j * 4096));
#pragma unroll
        for (int i = 0; i < C::IN; ++i) {
          acc[i][j] = mfma32_scaled(fa[i][0], fb[0], acc[i][j], ea, eb[j]);
          acc[i][j] = mfma32_scaled(fa[i][1], fb[1], acc[i][j], ea, eb[j]);
          const int ch = j * C::IN + i;
          if (SPREAD && ch * PER < C::LOADS) issue_rows(kn, nst, ch * PER, ch + 1 == C::IN * C::JM ? C::LOADS : (ch + 1) * PER);
        }
      }
      cur = (cur + 1 == S) ? 0 : cur + 1;
    }
  } else {
  // Software pipeline.  The 32x32 sub-tiles of a step are taken as chains c = j*IN + i
  // (two MFMAs each: K halves 0 and 1).  Each chain's MFMAs are issued before the
  // previous chain's promotion FMAs.  The last chain of a step is issued after the next
  // step's barrier, so the matrix core has work while that step's first fragment reads
  // are in flight; its operands stay in registers the new step's first reads do not touch.
  constexpr int CH = C::IN * C::JM;
  static_assert(CH % 2 == 0, "chains alternate between two result registers");
  v16f P[2];
  v8i fa[C::IN][2];
  v8i fb[2][2];
  float pc = 0.0f;   // scale product of the deferred chain
  auto promote = [&](int slot, int i, int j, float c) { acc[i][j] = P[slot] * c + acc[i][j]; };
  auto chain = [&](int slot, int i, int bslot) {
    P[slot] = mfma32(fa[i][0], fb[bslot][0], v16f{});
    P[slot] = mfma32(fa[i][1], fb[bslot][1], P[slot]);
  };

  constexpr int S = C::STAGES;
#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < nsteps) issue(kblock(p), p);
  int cur = 0;  // stage of step ks
  for (int ks = 0; ks < nsteps; ++ks) {
    // K groups: a step past this group's last K block adds nothing (zero scale product)
    const float live = (C::KSPLIT == 1 || ks * C::KSPLIT + grp < kblocks) ? 1.0f : 0.0f;
    // this thread's copies for step ks have landed (those of up to S-2 later steps may
    // still be in flight); after the barrier every thread's have, and no wave still
    // reads the stage the copies issued next overwrite
    if (ks + S - 2 < nsteps) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((S - 2) * C::VM_PER_STEP) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    const uint8_t FP8Q_LDS* st = lds + cur * C::STAGE_BYTES;
    const uint8_t FP8Q_LDS* stw = st + wn * 128;
    const uint8_t FP8Q_LDS* stt = st + (C::BN + wm) * 128;
    auto read_a = [&](int i) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        fa[i][h] = join(lds_ld<u32x4>(stw, fo[h][0] + i * 4096), lds_ld<u32x4>(stw, fo[h][1] + i * 4096));
    };
    auto read_b = [&](int j) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        fb[j & 1][h] = join(lds_ld<u32x4>(stt, fo[h][0] + j * 4096), lds_ld<u32x4>(stt, fo[h][1] + j * 4096));
    };
    read_b(0);
#pragma unroll
    for (int i = 0; i + 1 < C::IN; ++i) read_a(i);
    __builtin_amdgcn_sched_barrier(0);
    if (ks > 0) chain(1, C::IN - 1, (C::JM - 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    read_a(C::IN - 1);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = ks + S - 1 < nsteps;
    const int nst = cur == 0 ? S - 1 : cur - 1;  // the stage step ks+S-1 fills
    const int kn = kblock(more ? ks + S - 1 : nsteps - 1);
    if constexpr (SPREAD) {
      if (more) issue_scales(kn, nst);
    } else {
      if (more) issue(kn, nst);
    }
    __builtin_amdgcn_sched_barrier(0);
    float sa[C::JM];
    if constexpr (C::JM == 4) {
      const u32x4 t = lds_ld<u32x4>(st, so);
      sa[0] = __uint_as_float(t.x); sa[1] = __uint_as_float(t.y);
      sa[2] = __uint_as_float(t.z); sa[3] = __uint_as_float(t.w);
    } else if constexpr (C::JM == 2) {
      const u32x2 t = lds_ld<u32x2>(st, so);
      sa[0] = __uint_as_float(t.x); sa[1] = __uint_as_float(t.y);
    } else {
      sa[0] = lds_ld<float>(st, so);
    }
    const float sb = C::KSPLIT == 1 ? lds_ld<float>(st, wso) : lds_ld<float>(st, wso) * live;
    __builtin_amdgcn_sched_barrier(0);

    float c_prev = pc;
#pragma unroll
    for (int j = 0; j < C::JM; ++j) {
      const float c = sa[j] * sb;
#pragma unroll
      for (int i = 0; i < C::IN; ++i) {
        const int ch = j * C::IN + i;
        if (ch == CH - 1) break;  // deferred to the next step
        // a wave issuing MFMAs goes ahead of one issuing copies or promotion FMAs on the
        // same SIMD (4096^3: 74 -> 70 us; the power-of-two loop, which has no promotion
        // FMAs, measured no gain from it)
        __builtin_amdgcn_s_setprio(1);
        chain(ch & 1, i, j & 1);
        __builtin_amdgcn_s_setprio(0);
        if (SPREAD && ch * PER < C::LOADS) issue_rows(kn, nst, ch * PER, (ch + 1) * PER);
        if (i == 0 && j + 1 < C::JM) read_b(j + 1);
        if (ch > 0) {
          const int pi = (i == 0) ? C::IN - 1 : i - 1;
          const int pj = (i == 0) ? j - 1 : j;
          promote((ch - 1) & 1, pi, pj, (i == 0) ? c_prev : c);
        } else if (ks > 0) {
          promote(1, C::IN - 1, C::JM - 1, pc);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      c_prev = c;
    }
    if (SPREAD && (CH - 1) * PER < C::LOADS) issue_rows(kn, nst, (CH - 1) * PER, C::LOADS);
    // the deferred chain's operands fa[IN-1], fb[(JM-1)&1] are already in flight
    pc = sa[C::JM - 1] * sb;
    if (CH >= 2) promote((CH - 2) & 1, (CH - 2) % C::IN, (CH - 2) / C::IN, (C::IN == 1) ? sa[C::JM - 2] * sb : pc);
    __builtin_amdgcn_sched_barrier(0);
    cur = (cur + 1 == S) ? 0 : cur + 1;
  }
  if (nsteps > 0) {
    chain(1, C::IN - 1, (C::JM - 1) & 1);
    promote(1, C::IN - 1, C::JM - 1, pc);
  }
  if constexpr (C::KSPLIT > 1) {
    // the groups' partial sums, added in group order: group g > 0 writes its sums (lane-
    // contiguous, so every write and read covers whole bank rows), group 0 adds them
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    float FP8Q_LDS* red = reinterpret_cast<float FP8Q_LDS*>(lds0 + C::RED_OFF);
    constexpr int PER_WAVE = C::IN * C::JM * 16 * 64;
    if (grp > 0) {
      float FP8Q_LDS* dst = red + ((grp - 1) * C::GW + wave) * PER_WAVE + lane;
#pragma unroll
      for (int i = 0; i < C::IN; ++i)
#pragma unroll
        for (int j = 0; j < C::JM; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) dst[((i * C::JM + j) * 16 + e) * 64] = acc[i][j][e];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (grp == 0) {
#pragma unroll 1
      for (int g = 1; g < C::KSPLIT; ++g) {
        const float FP8Q_LDS* srcp = red + ((g - 1) * C::GW + wave) * PER_WAVE + lane;
#pragma unroll
        for (int i = 0; i < C::IN; ++i)
#pragma unroll
          for (int j = 0; j < C::JM; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] += srcp[((i * C::JM + j) * 16 + e) * 64];
      }
    }
  }

  }
  // ---- epilogue.  A lane holds y[m][n .. n+3] for m = wm + 32j + l%32 and
  // n = wn + 32i + 8q + 4(l/32): four outputs of one row per 8 bytes.  Each wave
  // rounds them to bf16 (once) into its own TM x TN row-major block of LDS, then reads
  // the block back in 16-byte row pieces, so that each global store instruction writes
  // whole row segments of 2*TN bytes.  16-byte chunks are XOR-swizzled per row so that
  // both the 8-byte writes and the 16-byte reads touch every LDS bank once per pass.
  constexpr int CPR = C::TN / 8;          // 16-byte chunks per row
  constexpr int RPW = 16 / CPR;           // rows per 256-byte bank window
  constexpr int RPI = 64 / CPR;           // rows per wave store instruction
  static_assert(C::GW * C::TM * C::TN * 2 <= C::LDS_BYTES, "epilogue staging fits in LDS");
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (grp > 0) return;  // K groups: group 0 holds the sums
  uint8_t FP8Q_LDS* ep = lds0 + wave * (C::TM * C::TN * 2);
#pragma unroll
  for (int j = 0; j < C::JM; ++j)
#pragma unroll
    for (int i = 0; i < C::IN; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int row = 32 * j + r32;
        const int chunk = (4 * i + q4) ^ ((row / RPW) & (CPR - 1));
        u32x2 o;
        o.x = bf16_rne(acc[i][j][4 * q4 + 0]) | (bf16_rne(acc[i][j][4 * q4 + 1]) << 16);
        o.y = bf16_rne(acc[i][j][4 * q4 + 2]) | (bf16_rne(acc[i][j][4 * q4 + 3]) << 16);
        *reinterpret_cast<u32x2 FP8Q_LDS*>(ep + row * (C::TN * 2) + chunk * 16 + 8 * g) = o;
      }
  if constexpr (SW) {
    // every wave's block is staged; 8 lanes per tile row take its 128 outputs, 16 each:
    // gate values from the wave block of columns 16cc.., up values from the block 128
    // columns further, both at the row's swizzled chunks 2(cc % 4) and 2(cc % 4) + 1
    __syncthreads();
    const int cc = lane & 7;
#pragma unroll 1
    for (int p = 0; p < C::BM / 64; ++p) {
      const int r = p * 64 + (tid >> 3);
      const int lr = r % C::TM, x = (lr / RPW) & (CPR - 1), c0 = 2 * (cc % 4);
      const uint8_t FP8Q_LDS* gb = lds + ((r / C::TM) * 4 + cc / 4) * (C::TM * C::TN * 2) + lr * (C::TN * 2);
      const uint8_t FP8Q_LDS* ub = gb + 2 * (C::TM * C::TN * 2);
      const u32x4 g0 = *reinterpret_cast<const u32x4 FP8Q_LDS*>(gb + ((c0 ^ x) << 4));
      const u32x4 g1 = *reinterpret_cast<const u32x4 FP8Q_LDS*>(gb + (((c0 + 1) ^ x) << 4));
      const u32x4 u0 = *reinterpret_cast<const u32x4 FP8Q_LDS*>(ub + ((c0 ^ x) << 4));
      const u32x4 u1 = *reinterpret_cast<const u32x4 FP8Q_LDS*>(ub + (((c0 + 1) ^ x) << 4));
      const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const uint32_t uw[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      const int64_t m = m0 + r;
      uint32_t o[4];
      float scale;
      if (swiglu_quant16<POW2>(gw, uw, m < m_end, o, scale)) {
        if (cc == 0) sw.s[jt * sw.ld_s + m] = scale;
        store_plain(sw.q + m * sw.ld_q + jt * 128 + cc * 16, make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
    return;
  }
  const int c_in = lane % CPR;
#pragma unroll
  for (int t = 0; t < C::TM / RPI; ++t) {
    const int row = t * RPI + lane / CPR;
    const u32x4 v = *reinterpret_cast<const u32x4 FP8Q_LDS*>(ep + row * (C::TN * 2) +
                                                           ((c_in ^ ((row / RPW) & (CPR - 1))) * 16));
    const int64_t m = m0 + wm + row;
    if (m < m_end) *reinterpret_cast<u32x4*>(y + m * ld_y + n0 + wn + 8 * c_in) = v;
  }
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
// Tile shapes.  Two waves per SIMD (8 per workgroup; 4 for the smallest tile): one
// wave's promotion FMAs and fragment reads overlap the other's MFMAs.  The large tile
// halves operand traffic per FLOP but leaves room in LDS for only two stages; the
// smaller tiles keep three steps of copies in flight, which their shorter steps need.
using CfgLarge = GemmCfg<256, 256, 2, 4, 2>;   // 128 x 64 per wave, 132 KB LDS
using CfgLargeHalf = GemmCfg<128, 256, 2, 4, 2>;  // 64 x 64 per wave: a group's last <= 128 rows
using CfgMid = GemmCfg<128, 128, 2, 4, 4>;     // 64 x 32 per wave, 132 KB LDS
using CfgMid2 = GemmCfg<128, 128, 2, 4, 2>;    // two workgroups per CU when tiles are plenty
using CfgMid2W4 = GemmCfg<128, 128, 2, 2, 2>;  // the same with 4 waves of 64 x 64
using CfgSmall = GemmCfg<128, 64, 2, 2, 4>;    // 64 x 32 per wave, 100 KB LDS
using CfgSmallK2 = GemmCfg<128, 64, 2, 2, 3, 2>;  // two K groups of 4 waves, 3-stage rings, 150 KB LDS

template <class C, bool POW2>
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
  gemm_tile<C, POW2>(a, ld_a, m, as, ld_as, b, ld_b, bs, kblocks, y, ld_y, m0, m_end, tn * C::BN,
               (uint8_t FP8Q_LDS*)lds);
}


// Ping-pong 256x256 tile for power-of-two scales.  The 8 waves form two groups of 4, each
// owning 128 token rows x 256 weight rows (128 x 64 per wave, as in CfgLarge).  A step is
// a memory phase (read every fragment of the K block into registers, start the next
// block's copies) and a compute phase (16 scaled MFMAs, nothing else).  The groups run
// half a step apart, one barrier out of phase: while one group computes, the other reads
// LDS, so the matrix core and LDS are busy at the same time instead of in bursts shared
// by all 8 waves.  Only power-of-two scales leave room for it: the fp32-scale tile's
// per-chain partial products (32 more registers) do not fit beside a whole step of
// fragments.  Copy rings: group 0 copies the weight rows (two stages shared by both
// groups), each group its own token rows and scales (two stages per group).
// Summation order per output is that of gemm_tile<CfgLarge, true>: K blocks in order,
// K halves 0 and 1 within a block; the results are bit-identical.
struct PingPongCfg {
  static constexpr int W_STAGE = 256 * 128;        // a step's 256 weight rows
  static constexpr int T_SCALE = 128 * 128;        // token scales, after a group's 128 rows
  static constexpr int T_WSC = T_SCALE + 128 * 4;  // per wave: the tile's two weight scales
  static constexpr int T_STAGE = 17408;
  static constexpr int T_BASE = 2 * W_STAGE;
  static constexpr int LDS_BYTES = T_BASE + 4 * T_STAGE;
};
static_assert(PingPongCfg::T_WSC + 4 * 8 <= PingPongCfg::T_STAGE && PingPongCfg::LDS_BYTES <= 160 * 1024 &&
                  8 * 128 * 64 * 2 <= PingPongCfg::LDS_BYTES,
              "ping-pong LDS: stages, and the epilogue's 8 wave blocks");

__device__ __forceinline__ void gemm_tile_pingpong_pow2(const uint8_t* __restrict__ a, int64_t ld_a,
                                                        int64_t a_rows, const float* __restrict__ as,
                                                        int64_t ld_as, const uint8_t* __restrict__ b,
                                                        int64_t ld_b, const float* __restrict__ bs, int kblocks,
                                                        uint16_t* __restrict__ y, int64_t ld_y, int64_t m0,
                                                        int64_t m_end, int64_t n0, uint8_t FP8Q_LDS* lds) {
  using Q = PingPongCfg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = wave >> 2, w4 = wave & 3;  // group; wave within it
  const int wn = w4 * 64;
  const int64_t tm0 = m0 + G * 128;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // Row copies: lane l of wave w4 copies chunk l%8 of rows 8*w4 + l/8 + 32i (weights: i < 8,
  // group 0 only; tokens: i < 4, clamped to the last valid row), swizzled as in gemm_tile.
  const int rl = w4 * 8 + (lane >> 3);
  const int chunk = (lane & 7) ^ swz(rl);  // swz(rl + 32i) == swz(rl)
  const uint32_t wsrc = (uint32_t)((n0 + rl) * ld_b) + chunk * 16;
  const uint32_t wstride = (uint32_t)(32 * ld_b);
  const uint32_t tsrc0 = (uint32_t)((tm0 + rl) * ld_a) + chunk * 16;
  const uint32_t tclamp = (uint32_t)((m_end - 1) * ld_a) + chunk * 16;
  const uint32_t tstride = (uint32_t)(32 * ld_a);
  // Scales: lanes 0..31 copy token scales into slots w4*32 + l (slot p holds token row
  // 32 * (p % 4) + p / 4 of the group, so a lane's four scales are contiguous); lanes 32
  // and 33 copy the tile's two weight scales into the wave's own pair of slots.
  const bool tok_lane = lane < 32;
  const int slot = w4 * 32 + (lane & 31);
  int64_t srow = tm0 + 32 * (slot & 3) + (slot >> 2);
  srow = srow < m_end ? srow : m_end - 1;
  const bool wsc_lane = lane == 32 || lane == 33;
  const uint32_t scsrc = tok_lane ? (uint32_t)(srow * 4) : (uint32_t)((n0 / 128 + (lane & 1)) * kblocks * 4);

  const v4i ra = make_rsrc(a, (uint32_t)(a_rows * ld_a));
  const v4i rb = make_rsrc(b, (uint32_t)((n0 + 256) * ld_b));
  const v4i rsa = make_rsrc(as, (uint32_t)(ld_as * kblocks * 4));
  const v4i rsb = make_rsrc(bs, (uint32_t)((n0 / 128 + 2) * kblocks * 4));

  auto issue = [&](int kb, int st) {
    const uint32_t tdst = lds_base + Q::T_BASE + (uint32_t)((G * 2 + st) * Q::T_STAGE);
    if (G == 0) {
      const uint32_t wdst = lds_base + (uint32_t)(st * Q::W_STAGE);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma16(rb, wsrc, (uint32_t)kb * 128u + (uint32_t)i * wstride, wdst + (uint32_t)((i * 4 + w4) * 1024));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = tsrc0 + (uint32_t)i * tstride;
      dma16(ra, o < tclamp ? o : tclamp, (uint32_t)kb * 128u, tdst + (uint32_t)((i * 4 + w4) * 1024));
    }
    if (tok_lane) dma4(rsa, scsrc, (uint32_t)(kb * ld_as * 4), tdst + Q::T_SCALE + (uint32_t)(w4 * 128));
    if (wsc_lane) dma4(rsb, scsrc, (uint32_t)kb * 4u, tdst + Q::T_WSC + (uint32_t)(w4 * 8) - 128u);
  };

  const int r32 = lane & 31, g = lane >> 5;
  uint32_t fo[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 2; ++e) fo[h][e] = (uint32_t)(r32 * 128 + (((4 * h + 2 * g + e) ^ swz(r32)) << 4));

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  v8i fa[2][2];  // weight fragments [sub-tile][K half]
  v8i fb[4][2];  // token fragments

  // Barriers: every wave passes 2 + 2 * kblocks before the epilogue's; group 1 takes its
  // extra one first (so it trails by one), group 0 last.  Between consecutive barriers
  // one group is in its memory phase and the other in its compute phase.  A stage is
  // rewritten only after both groups' reads of it have completed (lgkmcnt(0) before the
  // barrier that ends each memory phase), and a group's copies have landed (vmcnt(0)
  // before the barrier that ends its compute phase) before any wave reads them.
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  if (G == 1) asm volatile("s_barrier" ::: "memory");
  for (int s = 0; s < kblocks; ++s) {
    const int cur = s & 1;
    const uint8_t FP8Q_LDS* stw = lds + cur * Q::W_STAGE + wn * 128;
    const uint8_t FP8Q_LDS* stt = lds + Q::T_BASE + (G * 2 + cur) * Q::T_STAGE;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        fa[i][h] = join(lds_ld<u32x4>(stw, fo[h][0] + i * 4096), lds_ld<u32x4>(stw, fo[h][1] + i * 4096));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        fb[j][h] = join(lds_ld<u32x4>(stt, fo[h][0] + j * 4096), lds_ld<u32x4>(stt, fo[h][1] + j * 4096));
    const u32x4 t4 = lds_ld<u32x4>(stt, Q::T_SCALE + r32 * 16);
    const int ea = e8m0_of(lds_ld<float>(stt, Q::T_WSC + (w4 * 2 + (wn >> 7)) * 4));
    const int eb[4] = {(int)(t4.x >> 23), (int)(t4.y >> 23), (int)(t4.z >> 23), (int)(t4.w >> 23)};
    if (s + 1 < kblocks) issue(s + 1, cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // K half 0 of all 8 sub-tiles, then half 1: no MFMA waits for the one just before it
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) acc[i][j] = mfma32_scaled(fa[i][h], fb[j][h], acc[i][j], ea, eb[j]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  if (G == 0) asm volatile("s_barrier" ::: "memory");

  // epilogue as in gemm_tile: each wave stages its 128 x 64 bf16 block in LDS, swizzled,
  // and stores whole 128-byte row segments
  constexpr int TM = 128, TN = 64;
  constexpr int CPR = TN / 8, RPW = 16 / CPR, RPI = 64 / CPR;
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  uint8_t FP8Q_LDS* ep = lds + wave * (TM * TN * 2);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int row = 32 * j + r32;
        const int ck = (4 * i + q4) ^ ((row / RPW) & (CPR - 1));
        u32x2 o;
        o.x = bf16_rne(acc[i][j][4 * q4 + 0]) | (bf16_rne(acc[i][j][4 * q4 + 1]) << 16);
        o.y = bf16_rne(acc[i][j][4 * q4 + 2]) | (bf16_rne(acc[i][j][4 * q4 + 3]) << 16);
        *reinterpret_cast<u32x2 FP8Q_LDS*>(ep + row * (TN * 2) + ck * 16 + 8 * g) = o;
      }
  const int c_in = lane % CPR;
#pragma unroll
  for (int t = 0; t < TM / RPI; ++t) {
    const int row = t * RPI + lane / CPR;
    const u32x4 v = *reinterpret_cast<const u32x4 FP8Q_LDS*>(ep + row * (TN * 2) +
                                                           ((c_in ^ ((row / RPW) & (CPR - 1))) * 16));
    const int64_t m = tm0 + row;
    if (m < m_end) *reinterpret_cast<u32x4*>(y + m * ld_y + n0 + wn + 8 * c_in) = v;
  }
}

__global__ __launch_bounds__(512) void gemm_w8a8_pingpong_pow2_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, int64_t ld_b, const float* __restrict__ bs, uint16_t* __restrict__ y,
    int64_t ld_y, int64_t m, int64_t m_tiles, int64_t n_tiles, int kblocks) {
  __shared__ __align__(1024) uint8_t lds[PingPongCfg::LDS_BYTES];
  const int64_t tiles = m_tiles * n_tiles;
  const int64_t t = xcd_tile(blockIdx.x, tiles);
  if (t >= tiles) return;
  int64_t tm, tn;
  tile_coords<4>(t, m_tiles, n_tiles, tm, tn);
  const int64_t m0 = tm * 256;
  const int64_t m_end = (m0 + 256) < m ? (m0 + 256) : m;
  gemm_tile_pingpong_pow2(a, ld_a, m, as, ld_as, b, ld_b, bs, kblocks, y, ld_y, m0, m_end, tn * 256,
                          (uint8_t FP8Q_LDS*)lds);
}

template <class C, bool POW2 = false>
static hipError_t launch_dense(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                               int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                               int64_t k, hipStream_t stream) {
  const int64_t n_tiles = n / C::BN;
  const int64_t m_tiles = (m + C::BM - 1) / C::BM;
  const int64_t tiles = m_tiles * n_tiles;
  const int64_t grid = ((tiles + kXcds - 1) / kXcds) * kXcds;
  hipLaunchKernelGGL((gemm_w8a8_kernel<C, POW2>), dim3((unsigned)grid), dim3(C::THREADS), 0, stream,
                     reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b),
                     ld_b, b_s, reinterpret_cast<uint16_t*>(y), ld_y, m, m_tiles, n_tiles, (int)(k / 128));
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Few tokens (decode, short prefill): the GEMM streams the weight matrix once and is
// HBM-bound, so it is spread over as many CUs as possible.  A workgroup owns 16, 32 or 48
// weight rows and up to 16*WM token rows; its 8 waves take the K blocks round-robin.
// For each K block a wave loads the weight rows (non-temporal) and its live token rows
// (from L2) with 8 lanes per 128-byte line, writes them to its own LDS stage and reads
// them back in the MFMA operand layout, while the loads of its next K block are in flight.
// (Fragment loads straight from memory make every 16-lane quarter-wave touch 16 lines;
// measured on these shapes they move the same bytes about 1.6x slower.)  A stage row is
// 128 bytes with 16-byte chunk c of row r at c ^ ((r >> 1) & 7): the 16 lanes served
// together by a 16-byte LDS access then cover all 64 banks, both in a row-wise write (two
// whole rows) and in a fragment read (one chunk of each of 16 rows: rows 2i and 2i+1 share
// the chunk position and lie in the two halves of the 256-byte bank window).  The 8
// partial sums are added through LDS in a fixed order, so the result does not depend on
// timing.
//
// FUSED: the token rows arrive as bf16 and are quantized where they are loaded (FP8-RL
// summary page, "Method step details" step 1: activations are quantized dynamically on
// every forward).  Only the tile's live rows are quantized: 16 lanes per row take 8
// values each of the K block's 128-wide group, the group amax is the maximum over those
// 16 lanes, and the scale and codes follow the activation quantizer's rule with the same
// encoder, so the MFMA sees exactly the codes and scales a separate quantization would
// produce.  The codes go to the same stage rows, the scales beside them.
// ----------------------------------------------------------------------------
constexpr int kSmallWaves = 8;

// byte offset of 16-byte chunk c of row r in a stage
__device__ __forceinline__ int stage_at(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <int WM, bool FUSED, int D, int WN = 1, bool POW2 = false>
__global__ __launch_bounds__(64 * kSmallWaves) void gemm_smallm_kernel(
    const void* __restrict__ a_, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, int64_t ld_b, const float* __restrict__ bs, uint16_t* __restrict__ y,
    int64_t ld_y, int64_t m, int64_t n16, int kblocks) {
  constexpr int RT = 16 * WM;                                    // token rows of the tile
  constexpr int RW = 16 * WN;                                    // weight rows of the tile
  constexpr int kStage = (RW + RT) * 128 + (FUSED ? RT * 4 : 0);  // weight rows, token rows, scales
  constexpr int TP = RT / 8;                                     // row-wise token loads per lane
  constexpr int P = 4 * WM;                                      // FUSED: 64-lane passes over a tile's chunks
  static_assert(kStage >= WN * WM * 64 * 16, "the partial sums reuse the stage");
  __shared__ __align__(16) uint8_t stages[kSmallWaves * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint8_t* wst = stages + wave * kStage;
  uint8_t* tst = wst + RW * 128;
  float* sst = reinterpret_cast<float*>(wst + (RW + RT) * 128);
  const int64_t tn = blockIdx.x % n16;
  const int64_t m0 = (blockIdx.x / n16) * RT;
  const int64_t n0 = tn * RW;
  const int q = lane >> 4;
  const int fr = lane & 15;  // fragment row
  const int lr = lane >> 3, lc = lane & 7;  // row-wise lanes: row lr (+8i), chunk lc
  const int rows_live = (int)((m - m0) < RT ? (m - m0) : RT);
  const int chunks = rows_live * 16;  // FUSED: 8-value chunks of the live rows
  const uint8_t* a = reinterpret_cast<const uint8_t*>(a_);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a_);
  const uint8_t* w0 = b + (n0 + lr) * ld_b + lc * 16;
  const uint8_t* w1 = w0 + 8 * ld_b;
  int64_t srow[WM];  // token row of this lane's fragments (row 0 stands in for rows past m)
#pragma unroll
  for (int j = 0; j < WM; ++j) {
    const int r = 16 * j + fr;
    srow[j] = m0 + (r < rows_live ? r : 0);
  }

  // D K blocks in registers: slot d holds the wave's d-th, (d + D)-th, ... K block
  u32x4 rw[D][2 * WN];
  uint4 rt[D][FUSED ? P : TP];
  // weight scales: one per 16-row block where a tile can straddle two 128-row blocks
  constexpr int NSB = (128 % RW) ? WN : 1;
  float rsa[D][FUSED ? 1 : WM], rsb[D][NSB];
  auto load = [&](int d, int kb) {
#pragma unroll
    for (int wb = 0; wb < WN; ++wb) {
      const int64_t o = (int64_t)wb * 16 * ld_b + (int64_t)kb * 128;
      rw[d][2 * wb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w0 + o));
      rw[d][2 * wb + 1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(w1 + o));
    }
#pragma unroll
    for (int wb = 0; wb < NSB; ++wb) rsb[d][wb] = bs[((n0 + 16 * wb) / 128) * kblocks + kb];
    if constexpr (FUSED) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int c = p * 64 + lane;
        rt[d][p] = c < chunks ? load_plain(x + (m0 + c / 16) * ld_a + (int64_t)kb * 128 + (c % 16) * 8)
                              : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TP; ++i) {
        const int r = 8 * i + lr;
        rt[d][i] = r < rows_live
                       ? *reinterpret_cast<const uint4*>(a + (m0 + r) * ld_a + (int64_t)kb * 128 + lc * 16)
                       : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < WM; ++j) rsa[d][j] = as[(int64_t)kb * ld_as + srow[j]];
    }
  };

  v4f acc[WN][WM];
#pragma unroll
  for (int wb = 0; wb < WN; ++wb)
#pragma unroll
    for (int j = 0; j < WM; ++j) acc[wb][j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (wave + d * kSmallWaves < kblocks) load(d, wave + d * kSmallWaves);
  for (int kb0 = wave; kb0 < kblocks; kb0 += kSmallWaves * D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kb = kb0 + d * kSmallWaves;
      if (kb >= kblocks) break;
      // stage this K block
#pragma unroll
      for (int wb = 0; wb < WN; ++wb) {
        *reinterpret_cast<u32x4*>(wst + stage_at(16 * wb + lr, lc)) = rw[d][2 * wb];
        *reinterpret_cast<u32x4*>(wst + stage_at(16 * wb + lr + 8, lc)) = rw[d][2 * wb + 1];
      }
      float sa[WM];
      float sb[WN];
#pragma unroll
      for (int wb = 0; wb < WN; ++wb) sb[wb] = rsb[d][NSB > 1 ? wb : 0];
      if constexpr (FUSED) {
        // group amax over the 16 lanes of a row, then the activation quantizer's scale and
        // encoder; codes and scales into the stage
#pragma unroll
        for (int p = 0; p < P; ++p) {
          if (p * 64 >= chunks) break;
          const int c = p * 64 + lane;
          const uint4 v = rt[d][p];
          uint32_t mx = max_over_8_lanes(absmax8(v));
          mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x140, 0xf, 0xf, false));  // row mirror
          const float scale = POW2 ? scale_pow2_from_amax(bf16_bits_to_float(mx), kE4M3Max)
                                   : scale_from_amax(bf16_bits_to_float(mx), kE4M3Max);
          const Quantizer qz = make_quantizer(scale);
          const uint2 code = (qz.xm == 1.0f) ? quant8<false>(v, qz, false) : quant8<false>(v, qz, true);
          if (c < chunks) {
            const int r = c / 16, h = c % 16;
            *reinterpret_cast<uint2*>(tst + stage_at(r, h >> 1) + (h & 1) * 8) = code;
            if (h == 0) sst[r] = scale;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < TP; ++i) {
          const int r = 8 * i + lr;
          if (r < rows_live) *reinterpret_cast<uint4*>(tst + stage_at(r, lc)) = rt[d][i];
        }
#pragma unroll
        for (int j = 0; j < WM; ++j) sa[j] = rsa[d][j];
      }
      // this slot's next K block flies while this one is multiplied
      if (kb + kSmallWaves * D < kblocks) load(d, kb + kSmallWaves * D);
      __builtin_amdgcn_wave_barrier();
      v8i fw[WN];
#pragma unroll
      for (int wb = 0; wb < WN; ++wb)
        fw[wb] = join(*reinterpret_cast<const u32x4*>(wst + stage_at(16 * wb + fr, 2 * q)),
                      *reinterpret_cast<const u32x4*>(wst + stage_at(16 * wb + fr, 2 * q + 1)));
#pragma unroll
      for (int j = 0; j < WM; ++j) {
        const int r = 16 * j + fr;
        v8i ft = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        float s = 0.0f;
        if (r < rows_live) {
          ft = join(*reinterpret_cast<const u32x4*>(tst + stage_at(r, 2 * q)),
                    *reinterpret_cast<const u32x4*>(tst + stage_at(r, 2 * q + 1)));
          s = FUSED ? sst[r] : sa[j];
        }
#pragma unroll
        for (int wb = 0; wb < WN; ++wb) {
          const v4f p = mfma_fp8(fw[wb], ft);
          acc[wb][j] = p * (s * sb[wb]) + acc[wb][j];
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  // the partial sums go through the wave's own stage
  v4f* part = reinterpret_cast<v4f*>(wst);
#pragma unroll
  for (int wb = 0; wb < WN; ++wb)
#pragma unroll
    for (int j = 0; j < WM; ++j) part[(wb * WM + j) * 64 + lane] = acc[wb][j];
  __syncthreads();
  // wave w adds the 8 partial sums of sub-tiles w, w + 8, ... (sub-tile wb * WM + j) in a
  // fixed order and stores them
  for (int st = wave; st < WN * WM; st += kSmallWaves) {
    const int j = st % WM, wb = st / WM;
    v4f t = reinterpret_cast<const v4f*>(stages)[st * 64 + lane];
#pragma unroll
    for (int w = 1; w < kSmallWaves; ++w) t += reinterpret_cast<const v4f*>(stages + w * kStage)[st * 64 + lane];
    const int64_t row = m0 + 16 * j + (lane & 15);
    if (row < m) {
      const int64_t col = n0 + 16 * wb + 4 * q;
      uint2 o;
      o.x = bf16_rne(t[0]) | (bf16_rne(t[1]) << 16);
      o.y = bf16_rne(t[2]) | (bf16_rne(t[3]) << 16);
      *reinterpret_cast<uint2*>(y + row * ld_y + col) = o;
    }
  }
}

template <int WM, bool FUSED = false, int WN = 1, bool POW2 = false>
static hipError_t launch_smallm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                                int64_t k, hipStream_t stream) {
  const int64_t n16 = n / 16;
  const int64_t groups = (m + 16 * WM - 1) / (16 * WM);
  const unsigned grid = (unsigned)(n16 * groups);
  if constexpr (WN > 1) {
    hipLaunchKernelGGL((gemm_smallm_kernel<WM, FUSED, 1, WN, POW2>), dim3((unsigned)((n / (16 * WN)) * groups)),
                       dim3(64 * kSmallWaves), 0, stream, a, ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b),
                       ld_b, b_s, reinterpret_cast<uint16_t*>(y), ld_y, m, n / (16 * WN), (int)(k / 128));
    return hipGetLastError();
  }
  // K blocks in flight per wave: one, except two for a 16-token tile whose grid fits on the
  // CUs at once (measured: 1-4 tokens, N = K = 4096, 5.7 -> 4.9 us; deeper rings cost more in
  // occupancy than they gain wherever the grid is larger)
  if constexpr (!FUSED && WM == 1) {
    if (grid <= 256) {
      hipLaunchKernelGGL((gemm_smallm_kernel<WM, FUSED, 2>), dim3(grid), dim3(64 * kSmallWaves), 0, stream, a, ld_a,
                         a_s, ld_as, reinterpret_cast<const uint8_t*>(b), ld_b, b_s, reinterpret_cast<uint16_t*>(y),
                         ld_y, m, n16, (int)(k / 128));
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_smallm_kernel<WM, FUSED, 1, 1, POW2>), dim3(grid), dim3(64 * kSmallWaves), 0, stream, a, ld_a, a_s,
                     ld_as, reinterpret_cast<const uint8_t*>(b), ld_b, b_s, reinterpret_cast<uint16_t*>(y), ld_y, m,
                     n16, (int)(k / 128));
  return hipGetLastError();
}

// Token groups per workgroup for few tokens: 16*WM tokens, WM shrinking (more
// workgroups, each re-reading its weight rows from L2) until the grid covers every CU.
template <bool FUSED, bool POW2 = false>
static hipError_t launch_few_tokens(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                    int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                                    int64_t k, hipStream_t stream) {
  const int64_t n16 = n / 16;
  // 48 or 32 weight rows per workgroup where that still gives 192 workgroups or more: a
  // token row loaded into a workgroup then serves more weights, and the tokens, read once
  // per workgroup from L2, are most of the traffic.  Measured against 16 rows (interleaved,
  // byte-identical): 64x4096x4096 9.4 -> 8.3 us (32 tokens x 32 rows), 512x1024x4096
  // 13.1 -> 10.0 us (64 x 32), 256x1024x4096 8.0 -> 6.9 us; 64x12288x4096 24.6 -> 21.2 us
  // with 64 x 32 (384 workgroups: one and a half rounds of the CUs), 15.8 us with 64 x 48
  // (256), 32x12288x4096 15.1 -> 12.0 us with 32 x 48.  With 128 workgroups slower
  // (64x4096x4096 9.4 -> 11.0 us).
  // Fused activation quantization: every workgroup quantizes its token rows again, so 32
  // weight rows per workgroup halve that work (64 tokens x 32 rows spills; 32 x 32 and 16 x
  // 32 do not).  Interleaved medians, 16 -> 32 rows, byte-identical: 64x4096x4096 39.2 ->
  // 23.0 us, 33x4096x4096 25.4 -> 23.0, 64x12288x4096 113.2 -> 66.3, 16x12288x4096 27.5 ->
  // 20.6; with fewer than 192 workgroups no faster (16x4096x4096 12.9 -> 13.3).
  if constexpr (FUSED) {
    if (m > 16 && (n / 32) * ((m + 31) / 32) >= 192)
      return launch_smallm<2, FUSED, 2, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
    if (m > 8 && n / 32 >= 192)
      return launch_smallm<1, FUSED, 2, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  }
  if constexpr (!FUSED) {
    if (m > 32 && n % 48 == 0 && (n / 48) * ((m + 63) / 64) >= 192)
      return launch_smallm<4, FUSED, 3>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
    if (m > 32 && (n / 32) * ((m + 63) / 64) >= 192)
      return launch_smallm<4, FUSED, 2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
    if (m > 16 && n % 48 == 0 && (n / 48) * ((m + 31) / 32) >= 192)
      return launch_smallm<2, FUSED, 3>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
    if (m > 16 && (n / 32) * ((m + 31) / 32) >= 192)
      return launch_smallm<2, FUSED, 2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  }
  if (m > 32 && n16 >= 256)
    return launch_smallm<4, FUSED, 1, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  if (m > 16 && n16 * ((m + 31) / 32) >= 256)
    return launch_smallm<2, FUSED, 1, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  return launch_smallm<1, FUSED, 1, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
}

// FUSED with POW2: the tokens are quantized with the power-of-two rule, as the UE8M0
// activation quantizer would; the GEMM is the same promotion path (the products of
// power-of-two scales are the fp32 numbers the block-scaled MFMA would apply).
hipError_t launch_gemm_bf16act(const void* x, int64_t ld_x, const void* b, int64_t ld_b, const float* b_s, void* y,
                               int64_t ld_y, int64_t m, int64_t n, int64_t k, bool pow2, hipStream_t stream) {
  if (pow2) return launch_few_tokens<true, true>(x, ld_x, nullptr, 0, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  return launch_few_tokens<true>(x, ld_x, nullptr, 0, b, ld_b, b_s, y, ld_y, m, n, k, stream);
}

// Tile shape for M > 64 (POW2: the matrix core applies power-of-two block scales).
template <bool POW2>
static hipError_t launch_tiles(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                               int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                               int64_t k, hipStream_t stream) {
  if (m < 1024) {
    // two K groups per tile where each gets at least 4 steps (measured, interleaved medians:
    // 512x4096x4096 19.5 -> 17.1 us, 300x4096x12288 48.6 -> 39.3 us, 130x1024x4096 17.6 ->
    // 14.2 us; with 4-5 K steps in all the single group is faster: 700x1024x640 5.7 vs 6.1 us)
    if (!POW2 && k >= 1024)
      return launch_dense<CfgSmallK2, false>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
    return launch_dense<CfgSmall, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  }
  // large tiles when they cover n exactly and still give every CU a tile
  const int64_t large_tiles = ((m + CfgLarge::BM - 1) / CfgLarge::BM) * (n / CfgLarge::BN);
  if constexpr (POW2) {
    // ping-pong tile from 16 K steps on (interleaved medians, base -> ping-pong: 4096^3
    // 60.3 -> 57.2 us, 4096x12288x4096 164.6 -> 156.1, 8192^3 421 -> 396; even at
    // K = 1024, slower at K = 512: 8192x4096x512 28.0 -> 30.3)
    if (n % CfgLarge::BN == 0 && large_tiles >= 256 && k >= 2048) {
      const int64_t n_tiles = n / 256, m_tiles = (m + 255) / 256, tiles = m_tiles * n_tiles;
      const int64_t grid = ((tiles + kXcds - 1) / kXcds) * kXcds;
      hipLaunchKernelGGL(gemm_w8a8_pingpong_pow2_kernel, dim3((unsigned)grid), dim3(512), 0, stream,
                         reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b),
                         ld_b, b_s, reinterpret_cast<uint16_t*>(y), ld_y, m, m_tiles, n_tiles, (int)(k / 128));
      return hipGetLastError();
    }
  }
  if (n % CfgLarge::BN == 0 && large_tiles >= 256)
    return launch_dense<CfgLarge, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  // with at least two tiles per CU, two co-resident workgroups hide each other's waits
  // better than deeper copy rings
  const int64_t mid_tiles = ((m + CfgMid::BM - 1) / CfgMid::BM) * (n / CfgMid::BN);
  // Four waves of 64 x 64 read 25 % fewer LDS bytes per FLOP than eight of 64 x 32.
  // Interleaved medians, 8 -> 4 waves, byte-identical: power-of-two scales 4096x2048x4096
  // 40.6 -> 38.0 us, 2048x4096x4096 38.2 -> 36.5, 8192x1024x4096 42.6 -> 40.4, 65536x384x256
  // 20.7 -> 20.9; FP32 scales 4096x2048x4096 42.0 -> 40.8 and 40.4 -> 38.4, 2048x4096x4096
  // 41.8 -> 40.1, 4096x2048x2048 24.1 -> 23.2, but 8192x1024x4096 40.6 -> 41.8 and
  // 65536x384x256 19.1 -> 19.5, hence N >= 2048 there.
  if (mid_tiles >= 512 && (POW2 || n >= 2048))
    return launch_dense<CfgMid2W4, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  if (mid_tiles >= 512)
    return launch_dense<CfgMid2, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  return launch_dense<CfgMid, POW2>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
}

hipError_t launch_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                       int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                       int64_t k, bool pow2, hipStream_t stream) {
  // Few tokens, or few tiles: at most 64 tiles of 128x64 leave most CUs idle while each
  // tile walks all of K (a 128x64 tile takes about 14 us at K = 4096 however many run
  // beside it); the few-token kernel splits K over the 8 waves of every workgroup instead.
  // Measured on 56 shapes (80 <= m <= 700, n = 512 .. 4096, k = 1024 and 4096): with 64
  // tiles or fewer it was as fast or faster (130x1024x4096 13.9 -> 6.8 us, 256x512x4096
  // 14.0 -> 5.9 us), from 96 tiles slower.  Power-of-two scales take its promotion path too
  // (same result).
  const int64_t few_tiles = ((m + 127) / 128) * (n / 64);
  if (m <= 64 || (m < 1024 && k >= 1024 && few_tiles <= 64))
    return launch_few_tokens<false>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  if (pow2) return launch_tiles<true>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
  return launch_tiles<false>(a, ld_a, a_s, ld_as, b, ld_b, b_s, y, ld_y, m, n, k, stream);
}

// ----------------------------------------------------------------------------
// Grouped: rows of `a` are sorted by expert; rows [off[g], off[g+1]) use b[g].
// The tile schedule is derived on the device from the offsets: the grid is sized
// for the worst case (ceil(total_m / BM) + G m-tiles); each workgroup counts the
// m-tiles of the groups before it to find its (group, m-tile) and exits if it has
// none.  No host synchronization, no workspace.
// ----------------------------------------------------------------------------
// Grouped: the MoE layers give thousands of 128x128 tiles, so two co-resident
// workgroups per CU (measured faster than the four-stage ring here).
using CfgGrouped = CfgMid2;

// The (group, m-tile) of global m-tile `tile_m`: the groups' tiles, ceil(rows / BM) each,
// are numbered in group order; a 64-lane prefix sum per pass of 64 groups finds it.
// Wave 0 writes sel[0] = group (-1: none) and sel[1] = the tile within the group.
template <int BM>
__device__ __forceinline__ void find_group_tile(const int32_t* __restrict__ off, int32_t groups, int64_t tile_m,
                                                int32_t* sel) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t base = 0;
    int found_g = -1;
    int64_t found_t = 0;
    for (int g0 = 0; g0 < groups && found_g < 0; g0 += 64) {
      const int g = g0 + lane;
      int64_t tiles = 0;
      if (g < groups) tiles = (off[g + 1] - off[g] + BM - 1) / BM;
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
}

template <class C, bool POW2>
__global__ __launch_bounds__(C::THREADS) void grouped_gemm_w8a8_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, const float* __restrict__ bs, const int32_t* __restrict__ off,
    int32_t groups, uint16_t* __restrict__ y, int64_t ld_y, int64_t n, int64_t k, int64_t n_tiles) {
  __shared__ __align__(1024) uint8_t lds[C::LDS_BYTES];
  __shared__ int32_t sel[2];
  const int64_t tile_n = blockIdx.x % n_tiles;
  find_group_tile<C::BM>(off, groups, blockIdx.x / n_tiles, sel);
  const int g = sel[0];
  if (g < 0) return;
  const int kblocks = (int)(k / 128);
  const int64_t row0 = off[g] + (int64_t)sel[1] * C::BM;
  const int64_t row_end = (row0 + C::BM) < off[g + 1] ? (row0 + C::BM) : off[g + 1];
  const int64_t a_rows = off[groups];
  const uint8_t* bg = b + (int64_t)g * n * k;
  const float* bsg = bs + (int64_t)g * (n / 128) * kblocks;
  gemm_tile<C, POW2>(a, ld_a, a_rows, as, ld_as, bg, k, bsg, kblocks, y, ld_y, row0, row_end, tile_n * C::BN,
                     (uint8_t FP8Q_LDS*)lds);
}

// Two tile heights for the 256-wide tiles.  A group's rows are covered by 256-row tiles
// while more than 128 rows are left, and a remainder of at most 128 rows by one 128-row
// tile (a 94-row expert then runs 128 rows of MFMAs, not 256).  The global m-tile list
// holds every group's 256-row tiles in group order, then the 128-row tiles: the longer
// tiles are dispatched first.  Wave 0 writes sel[0] = group (-1: none), sel[1] = the
// tile's first row within the group, sel[2] = 1 for a 128-row tile.
__device__ __forceinline__ void find_group_tile_mixed(const int32_t* __restrict__ off, int32_t groups,
                                                      int64_t tile_m, int32_t* sel) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int found_g = -1, found_row = 0, small = 0;
    for (int pass = 0; pass < 2 && found_g < 0; ++pass) {
      int64_t base = 0;
      for (int g0 = 0; g0 < groups; g0 += 64) {
        const int g = g0 + lane;
        int64_t rows = g < groups ? (int64_t)(off[g + 1] - off[g]) : 0;
        const int64_t rem = rows & 255;
        const int64_t tiles = pass == 0 ? (rows >> 8) + (rem > 128) : (rem > 0 && rem <= 128);
        int64_t incl = tiles;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int64_t o = __shfl_up(incl, d);
          if (lane >= d) incl += o;
        }
        const int64_t excl = incl - tiles;
        const bool mine = tiles > 0 && tile_m >= base + excl && tile_m < base + incl;
        const unsigned long long hit = __ballot(mine);
        if (hit && found_g < 0) {
          const int src = __ffsll(hit) - 1;
          found_g = g0 + src;
          const int64_t t = tile_m - base - __shfl(excl, src);
          found_row = pass == 0 ? (int)(256 * t) : (int)(__shfl(rows, src) & ~(int64_t)255);
          small = pass;
        }
        base += __shfl(incl, 63);
      }
      tile_m -= base;  // the 128-row tiles are numbered after all 256-row tiles
    }
    if (lane == 0) {
      sel[0] = found_g;
      sel[1] = found_row;
      sel[2] = small;
    }
  }
  __syncthreads();
}

// 256-wide tiles of both heights in one grid (for K >= 2048; see launch_grouped_gemm)
template <bool POW2>
__global__ __launch_bounds__(CfgLarge::THREADS) void grouped_gemm_mixed_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, const float* __restrict__ bs, const int32_t* __restrict__ off,
    int32_t groups, uint16_t* __restrict__ y, int64_t ld_y, int64_t n, int64_t k, int64_t n_tiles) {
  static_assert(CfgLargeHalf::LDS_BYTES <= CfgLarge::LDS_BYTES && CfgLargeHalf::THREADS == CfgLarge::THREADS,
                "both tile heights share the launch");
  __shared__ __align__(1024) uint8_t lds[CfgLarge::LDS_BYTES];
  __shared__ int32_t sel[3];
  const int64_t tile_n = blockIdx.x % n_tiles;
  find_group_tile_mixed(off, groups, blockIdx.x / n_tiles, sel);
  const int g = sel[0];
  if (g < 0) return;
  const int kblocks = (int)(k / 128);
  const int64_t row0 = off[g] + sel[1];
  const int64_t a_rows = off[groups];
  const uint8_t* bg = b + (int64_t)g * n * k;
  const float* bsg = bs + (int64_t)g * (n / 128) * kblocks;
  if (sel[2] == 0) {
    const int64_t row_end = (row0 + 256) < off[g + 1] ? (row0 + 256) : off[g + 1];
    gemm_tile<CfgLarge, POW2>(a, ld_a, a_rows, as, ld_as, bg, k, bsg, kblocks, y, ld_y, row0, row_end,
                              tile_n * 256, (uint8_t FP8Q_LDS*)lds);
  } else {
    gemm_tile<CfgLargeHalf, POW2>(a, ld_a, a_rows, as, ld_as, bg, k, bsg, kblocks, y, ld_y, row0, off[g + 1],
                                  tile_n * 256, (uint8_t FP8Q_LDS*)lds);
  }
}

// MoE fc1 with SwiGLU and fc2's 1x128 quantization fused into the epilogue: B is
// [G][2 half][k] (gate rows, then up rows); tile column tn covers outputs 128tn .. +127.
template <bool POW2>
__global__ __launch_bounds__(CfgLarge::THREADS) void grouped_swiglu_kernel(
    const uint8_t* __restrict__ a, int64_t ld_a, const float* __restrict__ as, int64_t ld_as,
    const uint8_t* __restrict__ b, const float* __restrict__ bs, const int32_t* __restrict__ off,
    int32_t groups, int64_t half, int64_t k, int64_t n_tiles, uint8_t* __restrict__ q, int64_t ld_q,
    float* __restrict__ s, int64_t ld_s, const int32_t* __restrict__ row_token, int64_t token_rows) {
  __shared__ __align__(1024) uint8_t lds[CfgLarge::LDS_BYTES];
  __shared__ int32_t sel[3];
  const int64_t tile_n = blockIdx.x % n_tiles;
  find_group_tile_mixed(off, groups, blockIdx.x / n_tiles, sel);
  const int g = sel[0];
  if (g < 0) return;
  const int kblocks = (int)(k / 128);
  const int64_t row0 = off[g] + sel[1];
  const int64_t a_rows = row_token ? token_rows : off[groups];
  const uint8_t* bg = b + (int64_t)g * 2 * half * k;
  const float* bsg = bs + (int64_t)g * (2 * half / 128) * kblocks;
  SwigluOut so;
  so.q = q;
  so.ld_q = ld_q;
  so.s = s;
  so.ld_s = ld_s;
  so.half = half;
  if (sel[2] == 0) {
    const int64_t row_end = (row0 + 256) < off[g + 1] ? (row0 + 256) : off[g + 1];
    gemm_tile<CfgLarge, POW2, true>(a, ld_a, a_rows, as, ld_as, bg, k, bsg, kblocks, nullptr, 0, row0, row_end,
                                    tile_n * 256, (uint8_t FP8Q_LDS*)lds, so, row_token);
  } else {
    gemm_tile<CfgLargeHalf, POW2, true>(a, ld_a, a_rows, as, ld_as, bg, k, bsg, kblocks, nullptr, 0, row0,
                                        off[g + 1], tile_n * 256, (uint8_t FP8Q_LDS*)lds, so, row_token);
  }
}

template <class C>
static hipError_t launch_grouped(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                 const float* b_s, const int32_t* offsets, int32_t groups, int64_t total_m, void* y,
                                 int64_t ld_y, int64_t n, int64_t k, bool pow2, hipStream_t stream) {
  const int64_t n_tiles = n / C::BN;
  const int64_t m_tiles = (total_m + C::BM - 1) / C::BM + groups;
  auto kernel = pow2 ? grouped_gemm_w8a8_kernel<C, true> : grouped_gemm_w8a8_kernel<C, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)(n_tiles * m_tiles)), dim3(C::THREADS), 0, stream,
                     reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b), b_s,
                     offsets, groups, reinterpret_cast<uint16_t*>(y), ld_y, n, k, n_tiles);
  return hipGetLastError();
}

// Tile shape by K: with 16 or more K steps per tile the 256x256 tile's lower operand
// traffic per FLOP wins despite more padding in small experts (MoE fc1, 128 experts,
// K = 2048, median 94 rows per expert: 240 -> 213 us); with few K steps two co-resident
// 128x128 workgroups hide each other's prologue and epilogue (fc2, K = 768: 129 us vs 134).
hipError_t launch_grouped_swiglu(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                 const float* b_s, const int32_t* offsets, int32_t groups, int64_t total_m,
                                 int64_t half, int64_t k, void* q, int64_t ld_q, float* s, int64_t ld_s,
                                 const int32_t* row_token, int64_t token_rows, bool pow2, hipStream_t stream) {
  using C = CfgLarge;
  const int64_t n_tiles = half / 128;
  // 256-row tiles: at most total_m / 256 + one per group; 128-row tiles: at most one per group
  const int64_t m_tiles = (total_m + 255) / 256 + 2 * (int64_t)groups;
  auto kernel = pow2 ? grouped_swiglu_kernel<true> : grouped_swiglu_kernel<false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)(n_tiles * m_tiles)), dim3(C::THREADS), 0, stream,
                     reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b), b_s,
                     offsets, groups, half, k, n_tiles, reinterpret_cast<uint8_t*>(q), ld_q, s, ld_s, row_token,
                     token_rows);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                               const void* b, const float* b_s, const int32_t* offsets, int32_t groups,
                               int64_t total_m, void* y, int64_t ld_y, int64_t n, int64_t k, bool pow2,
                               hipStream_t stream) {
  if (k >= 16 * 128 && n % CfgLarge::BN == 0) {
    const int64_t n_tiles = n / 256;
    const int64_t m_tiles = (total_m + 255) / 256 + 2 * (int64_t)groups;  // as for the fused fc1
    auto kernel = pow2 ? grouped_gemm_mixed_kernel<true> : grouped_gemm_mixed_kernel<false>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(n_tiles * m_tiles)), dim3(CfgLarge::THREADS), 0, stream,
                       reinterpret_cast<const uint8_t*>(a), ld_a, a_s, ld_as, reinterpret_cast<const uint8_t*>(b),
                       b_s, offsets, groups, reinterpret_cast<uint16_t*>(y), ld_y, n, k, n_tiles);
    return hipGetLastError();
  }
  return launch_grouped<CfgGrouped>(a, ld_a, a_s, ld_as, b, b_s, offsets, groups, total_m, y, ld_y, n, k, pow2,
                                    stream);
}

}  // namespace fp8q


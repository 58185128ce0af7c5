// FP8 paged decode attention over the quantized KV cache, with per-step recalibration
// of the query scale, for gfx950.
//
// FP8-RL summary page, "Method step details" step 3: the Q/K/V scales are recomputed
// at the start of every RL step's rollout; "Experimental results": full FP8 rollout
// quantizes the linear layers, the KV cache and attention.  "1T-parameter RL on 100
// GPUs", 3.4: the cache is paged in fixed blocks.
//
// One decode query per sequence and query head.  The query is quantized to E4M3 with
// its own per-layer scale (the activation rule: a recalibrating call first sets it to
// fl32(amax / range) over the call's queries), so the scores are FP8 x FP8 products:
//   s_t = sm_scale * q_scale * k_scale * sum_d dec(cq[d]) * dec(ck[t][d]),
//   out[d] = v_scale * sum_t softmax(s)_t * dec(cv[t][d]).
// Softmax and the value sum run in fp32 on the exactly decoded codes; the output is
// rounded to bf16 once.
//
// The query-key products are products of E4M3 values, which bf16 holds exactly, so the
// matrix core computes them with bf16 MFMAs on the decoded codes: its FP8 MFMA
// accumulates with a relative error up to about 2^-12 of the sum of |products| (measured),
// enough to move the weights of a peaked softmax; the bf16 MFMA accumulates in fp32.
//
// A workgroup owns one (sequence, KV head) pair and the query heads that share it
// (grouped-query attention, up to 16).  Its 8 waves take 64-token chunks of the
// context round-robin.  Per chunk a wave runs, for each 16-token tile, four chained
// 16x16x32 bf16 MFMAs (A = 16 cached key rows, B = the group's query codes padded to 16
// columns; a lane's 32 contiguous dimensions are its K slots of the four), updates a running
// maximum and sum per head (online softmax), and adds p * V with fp32 FMAs: a lane owns
// 8 head dimensions of all the group's heads for the chunk's tokens t = quarter (mod 4),
// with the weights p read from LDS.  The waves' partial (max, sum, vector) triples are
// combined through LDS in a fixed order, so the result does not depend on timing.
// A chunk's key rows are loaded with 8 lanes per 128-byte row (a quarter-wave of MFMA
// fragment loads would touch 16 rows, which measured slower) and pass through a per-wave
// LDS stage laid out so that the 16 lanes served together by a 16-byte LDS access cover all
// 64 banks, both in the row-wise writes and in the fragment reads (key_slot); value rows
// already arrive as whole 128-byte lines per quarter-wave.
#include "e4m3.hpp"
#include "launch.hpp"

namespace fp8q {

typedef float att_v4f __attribute__((ext_vector_type(4)));
typedef __bf16 att_v8bf __attribute__((ext_vector_type(8)));
typedef unsigned int att_u32x4 __attribute__((ext_vector_type(4)));

// 8 E4M3 codes (two dwords) -> 8 bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ att_v8bf fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  att_u32x4 o;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w = h ? w1 : w0;
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    o[2 * h] = (__float_as_uint(lo[0]) >> 16) | (__float_as_uint(lo[1]) & 0xffff0000u);
    o[2 * h + 1] = (__float_as_uint(hi[0]) >> 16) | (__float_as_uint(hi[1]) & 0xffff0000u);
  }
  return __builtin_bit_cast(att_v8bf, o);
}

// LDS offset of 16-byte chunk c of key-stage row r (row = token * HG + head).  A fragment
// read takes one chunk of 16 rows of one head; the bank group of a 16-byte slot is the
// row's half of the 256-byte bank window and the chunk position.  HG = 1: rows 2i and 2i+1
// share the position c ^ ((r >> 1) & 7) and fill the two halves.  HG = 2: the rows read
// together have one parity, so rows are swapped in pairs (r ^ ((r >> 1) & 1)) to alternate
// the halves, with the position c ^ ((r >> 2) & 7).  A row-wise write (one or two tokens,
// whole rows) also covers every bank.
template <int HG>
__device__ __forceinline__ int key_slot(int r, int c) {
  static_assert(HG == 1 || HG == 2, "one or two KV heads per workgroup");
  if constexpr (HG == 1) return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
  return (r ^ ((r >> 1) & 1)) * 128 + ((c ^ ((r >> 2) & 7)) << 4);
}

constexpr int kAttnWaves = 8;
constexpr int kAttnChunk = 64;
constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------------------
// Query-scale recalibration: one workgroup reduces |q| over the call's queries and
// stores fl32(amax / range) (1 for amax 0).  Decode queries are small (sequences x
// heads x 128 values), so one workgroup and no atomics suffice.
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void q_scale_kernel(const uint16_t* __restrict__ q, int64_t ld_q, int64_t seqs,
                                                       int64_t row, float range, float* __restrict__ q_scale) {
  __shared__ uint32_t red[16];
  constexpr int U = 16;  // loads in flight per thread (one per trip serialises on latency)
  uint32_t mx = 0;
  const int64_t total = seqs * row;
  for (int64_t i0 = (int64_t)threadIdx.x * 8; i0 < total; i0 += 1024 * 8 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + (int64_t)u * 1024 * 8;
      const int64_t b = i / row;
      v[u] = i < total ? load_plain(q + b * ld_q + (i - b * row)) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) mx = max(mx, absmax8(v[u]));
  }
  mx = max_over_wave(mx);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    for (int w = 0; w < 16; ++w) m = max(m, red[w]);
    q_scale[0] = scale_from_amax(bf16_bits_to_float(m), range);
  }
}

// page and slot of token t (page_size a power of two: shift and mask)
struct PageMap {
  int32_t size, shift;  // shift < 0: not a power of two
  __device__ __forceinline__ void split(int t, int& page_idx, int& slot) const {
    if (shift >= 0) {
      page_idx = t >> shift;
      slot = t & (size - 1);
    } else {
      page_idx = t / size;
      slot = t - page_idx * size;
    }
  }
};

// PS16: 16-token pages, so a chunk is whole pages: the page ids are wave-uniform (scalar
// loads) and every lane's offset within a page is fixed.
// HG: KV heads per workgroup.  The cache keeps a token's KV heads side by side, so with
// HG = 2 every token contributes 256 contiguous bytes (a read of this cache with one head
// per workgroup measured 5.4 TB/s, with two 6.1 TB/s).  A chunk holds 64 / HG tokens, so a
// wave's loads per chunk stay at 16 KB.
template <int GMAX, bool PS16, int HG>
__global__ __launch_bounds__(64 * kAttnWaves) void paged_decode_attn_kernel(
    const uint16_t* __restrict__ q, int64_t ld_q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ bt, int64_t ld_bt, const int32_t* __restrict__ seq_lens, int32_t hkv,
    int32_t group, PageMap pm, const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, float sm_scale, uint16_t* __restrict__ out, int64_t ld_out) {
  constexpr int CT = kAttnChunk / HG;  // tokens per chunk
  constexpr int NT = CT / 16;          // 16-token score tiles per chunk
  constexpr int NV = CT / 4;           // value rows per lane, chunk and head
  constexpr int NP = (CT + 15) / 16;   // PS16: pages per chunk
  constexpr int TPI = 8 / HG;          // tokens per row-wise key load
  constexpr int GH = HG * GMAX;        // head slots of the workgroup
  __shared__ float pbuf[kAttnWaves][HG][CT][GMAX];  // a chunk's softmax weights
  __shared__ float abuf[kAttnWaves][GH];             // rescale factor of the running sums
  __shared__ float mred[kAttnWaves][GH], lred[kAttnWaves][GH];
  // per-wave key stages during the chunk loop, the waves' partial vectors after it
  constexpr int kKeyStage = CT * HG * 128;
  constexpr int kShared = kAttnWaves * (kKeyStage > GH * 128 * 4 ? kKeyStage : GH * 128 * 4);
  __shared__ __align__(16) uint8_t kshare[kShared];
  float(*ored)[GH][128] = reinterpret_cast<float(*)[GH][128]>(kshare);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hcol = lane & 15, quad = lane >> 4;
  const int hkg = hkv / HG;  // workgroups per sequence
  const int b = blockIdx.x / hkg, g0 = (blockIdx.x - (blockIdx.x / hkg) * hkg) * HG;
  const int L = seq_lens[b];
  const uint16_t* qb = q + (int64_t)b * ld_q + (int64_t)g0 * group * 128;
  uint16_t* ob = out + (int64_t)b * ld_out + (int64_t)g0 * group * 128;
  if (L <= 0) {
    for (int t = threadIdx.x; t < HG * group * 128; t += 64 * kAttnWaves) ob[t] = 0;
    return;
  }
  const int32_t* btb = bt + (int64_t)b * ld_bt;
  const float qs = q_scale[0], ks = k_scale[0], vs = v_scale[0];

  // query codes of KV head g0 + hh in the MFMA B layout: lane l holds head l % 16 of the
  // group (zero past it), dimensions 32 * (l / 16) + 8c .. +7 for MFMA c; codes saturate
  // (a stored scale may be exceeded)
  att_v8bf fq[HG][4];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    uint4 c0 = make_uint4(0, 0, 0, 0), c1 = c0;
    if (hcol < group) {
      const uint16_t* p = qb + (hh * group + hcol) * 128 + quad * 32;
      const Quantizer qz = make_quantizer(qs);
      c0 = quant16<true>(load_plain(p), load_plain(p + 8), qz);
      c1 = quant16<true>(load_plain(p + 16), load_plain(p + 24), qz);
    }
    fq[hh][0] = fp8x8_to_bf16(c0.x, c0.y);
    fq[hh][1] = fp8x8_to_bf16(c0.z, c0.w);
    fq[hh][2] = fp8x8_to_bf16(c1.x, c1.y);
    fq[hh][3] = fp8x8_to_bf16(c1.z, c1.w);
  }
  const float f = sm_scale * qs * ks * kLog2e;  // scores in log2 units

  float m_run[HG], l_run[HG];  // head hcol of each KV head's group
  float acc[HG][GMAX][8];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.0f;
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[hh][h][d] = 0.0f;
  }

  const int nchunks = (L + CT - 1) / CT;
  const int64_t page_bytes = (int64_t)pm.size * hkv * 128;
  // PS16 lane offsets within a page of value rows (token quad + 4r, dims 8*hcol..)
  int voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) voff[r] = ((quad + 4 * r) * hkv + g0) * 128 + hcol * 8;
  // row-wise key lanes: token kt (+TPI*u), 16-byte chunk kcol of the token's HG heads
  const int kt = lane / (8 * HG), kcol = lane % (8 * HG);
  const int kroff = (kt * hkv + g0) * 128 + kcol * 16;  // PS16: within a page
  uint8_t* kst = kshare + wave * kKeyStage;
  struct Chunk {
    uint4 kr[8];        // keys: token t0 + TPI*u + kt, bytes 16 * kcol .. +15 of its HG heads
    uint2 vr[HG][NV];   // values of head g0 + hh: tokens t0 + quad + 4j, dimensions 8 * hcol .. +7
  };
  auto load_chunk = [&](int c, Chunk& R) {
    const int t0 = c * CT;
    int64_t pbase[NP];
    if constexpr (PS16) {
#pragma unroll
      for (int i = 0; i < NP; ++i) pbase[i] = (t0 + 16 * i < L) ? (int64_t)btb[c * NP + i] * page_bytes : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + TPI * u + kt;
      R.kr[u] = make_uint4(0, 0, 0, 0);
      if (t < L) {
        const uint8_t* kp;
        if constexpr (PS16) {
          kp = kc + pbase[(TPI * u) / 16] + ((TPI * u) % 16) * hkv * 128 + kroff;
        } else {
          int pi, slot;
          pm.split(t, pi, slot);
          kp = kc + (((int64_t)btb[pi] * pm.size + slot) * hkv + g0) * 128 + kcol * 16;
        }
        R.kr[u] = load_plain(kp);
      }
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int t = t0 + quad + 4 * j;
        R.vr[hh][j] = make_uint2(0, 0);
        if (t < L) {
          const uint8_t* vp;
          if constexpr (PS16) {
            vp = vc + pbase[j / 4] + voff[j % 4] + hh * 128;
          } else {
            int pi, slot;
            pm.split(t, pi, slot);
            vp = vc + (((int64_t)btb[pi] * pm.size + slot) * hkv + g0 + hh) * 128 + hcol * 8;
          }
          R.vr[hh][j] = *reinterpret_cast<const uint2*>(vp);
        }
      }
  };
  auto compute_chunk = [&](int c, const Chunk& R) {
    const int t0 = c * CT;
    // key rows into the wave's stage (row = token * HG + head), then back in the MFMA
    // layout: tile i, lane row = token t0 + 16i + hcol, code bytes 32 * quad .. +31
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (TPI * u + kt) * HG + (kcol >> 3);
      *reinterpret_cast<uint4*>(kst + key_slot<HG>(row, kcol & 7)) = R.kr[u];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      // scores: lane holds head hcol, tokens t0 + 16i + 4 * quad + e
      float sc[NT][4];
      float mc = -INFINITY;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        const int row = (16 * i + hcol) * HG + hh;
        const uint4 k0 = *reinterpret_cast<const uint4*>(kst + key_slot<HG>(row, 2 * quad));
        const uint4 k1 = *reinterpret_cast<const uint4*>(kst + key_slot<HG>(row, 2 * quad + 1));
        att_v4f r = {0.f, 0.f, 0.f, 0.f};
        r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k0.x, k0.y), fq[hh][0], r, 0, 0, 0);
        r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k0.z, k0.w), fq[hh][1], r, 0, 0, 0);
        r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k1.x, k1.y), fq[hh][2], r, 0, 0, 0);
        r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16(k1.z, k1.w), fq[hh][3], r, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[i][e] = (t0 + 16 * i + 4 * quad + e < L) ? r[e] * f : -INFINITY;
          mc = fmaxf(mc, sc[i][e]);
        }
      }
      mc = fmaxf(mc, __shfl_xor(mc, 16));
      mc = fmaxf(mc, __shfl_xor(mc, 32));
      const float m_new = fmaxf(m_run[hh], mc);  // finite: the chunk holds a token below L
      const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - m_new);
      float ls = 0.0f;
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[i][e] = __builtin_amdgcn_exp2f(sc[i][e] - m_new);
          ls += sc[i][e];
        }
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      l_run[hh] = l_run[hh] * alpha + ls;
      m_run[hh] = m_new;
      // weights and rescale factors to LDS; the wave reads only what it wrote
      if (hcol < GMAX) {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) pbuf[wave][hh][16 * i + 4 * quad + e][hcol] = sc[i][e];
        if (quad == 0) abuf[wave][hh * GMAX + hcol] = alpha;
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float a = abuf[wave][hh * GMAX + h];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[hh][h][d] *= a;
      }
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int tl = quad + 4 * j;
        float v[8];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const uint32_t word = w ? R.vr[hh][j].y : R.vr[hh][j].x;
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
          v[4 * w + 0] = lo[0];
          v[4 * w + 1] = lo[1];
          v[4 * w + 2] = hi[0];
          v[4 * w + 3] = hi[1];
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          const float p = pbuf[wave][hh][tl][h];
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[hh][h][d] = __builtin_fmaf(p, v[d], acc[hh][h][d]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  for (int c = wave; c < nchunks; c += kAttnWaves) {
    Chunk R;
    load_chunk(c, R);
    compute_chunk(c, R);
  }
  // the four quarters of the chunk's tokens, then the waves (whose partial vectors reuse
  // the key stages: every wave has left its chunk loop before any is overwritten)
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < HG; ++hh)
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        acc[hh][h][d] += __shfl_xor(acc[hh][h][d], 16);
        acc[hh][h][d] += __shfl_xor(acc[hh][h][d], 32);
      }
  if (quad == 0) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int d = 0; d < 8; ++d) ored[wave][hh * GMAX + h][8 * hcol + d] = acc[hh][h][d];
      if (hcol < GMAX) {
        mred[wave][hh * GMAX + hcol] = m_run[hh];
        lred[wave][hh * GMAX + hcol] = l_run[hh];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < HG * group * 128; t += 64 * kAttnWaves) {
    const int hh = t / (group * 128);
    const int rem = t - hh * group * 128;
    const int slot = hh * GMAX + (rem >> 7), d = rem & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, mred[w][slot]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float e = __builtin_amdgcn_exp2f(mred[w][slot] - M);  // 0 for a wave without tokens
      num = __builtin_fmaf(e, ored[w][slot][d], num);
      den = __builtin_fmaf(e, lred[w][slot], den);
    }
    const uint32_t u = __float_as_uint(vs * (num / den));
    ob[t] = (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
}

hipError_t launch_decode_attention(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int64_t ld_bt, const int32_t* seq_lens, int32_t seqs,
                                   int32_t hq, int32_t hkv, int32_t page_size, float* q_scale, const float* k_scale,
                                   const float* v_scale, float sm_scale, float range, bool recalibrate, void* out,
                                   int64_t ld_out, hipStream_t stream) {
  if (recalibrate) {
    hipLaunchKernelGGL(q_scale_kernel, dim3(1), dim3(1024), 0, stream, reinterpret_cast<const uint16_t*>(q), ld_q,
                       (int64_t)seqs, (int64_t)hq * 128, range, q_scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (seqs == 0) return hipSuccess;
  PageMap pm;
  pm.size = page_size;
  pm.shift = ((page_size & (page_size - 1)) == 0) ? __builtin_ctz((unsigned)page_size) : -1;
  const int32_t group = hq / hkv;
  // two KV heads per workgroup: 256 contiguous bytes per token, while half as many
  // workgroups still cover the 256 CUs (measured, 64 sequences x 8 KV heads x 20,000 tokens:
  // 538 -> 521 us; 16 sequences: 38 -> 68 us, hence the grid condition); the pair's
  // registers fit for groups of up to 4 query heads
  const bool pair_heads = group <= 4 && hkv % 2 == 0 && (int64_t)seqs * hkv >= 512;
  const dim3 grid((unsigned)((int64_t)seqs * (pair_heads ? hkv / 2 : hkv))), block(64 * kAttnWaves);
  const auto* qp = reinterpret_cast<const uint16_t*>(q);
  const auto* kp = reinterpret_cast<const uint8_t*>(k_cache);
  const auto* vp = reinterpret_cast<const uint8_t*>(v_cache);
  auto* op = reinterpret_cast<uint16_t*>(out);
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, qp, ld_q, kp, vp, block_table, ld_bt, seq_lens, hkv, group,
                       pm, q_scale, k_scale, v_scale, sm_scale, op, ld_out);
  };
  const bool ps16 = page_size == 16;
  if (pair_heads)
    ps16 ? launch(paged_decode_attn_kernel<4, true, 2>) : launch(paged_decode_attn_kernel<4, false, 2>);
  else if (group <= 4)
    ps16 ? launch(paged_decode_attn_kernel<4, true, 1>) : launch(paged_decode_attn_kernel<4, false, 1>);
  else if (group <= 8)
    ps16 ? launch(paged_decode_attn_kernel<8, true, 1>) : launch(paged_decode_attn_kernel<8, false, 1>);
  else
    ps16 ? launch(paged_decode_attn_kernel<16, true, 1>) : launch(paged_decode_attn_kernel<16, false, 1>);
  return hipGetLastError();
}

}  // namespace fp8q

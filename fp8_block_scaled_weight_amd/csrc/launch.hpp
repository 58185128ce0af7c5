// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// One weight tensor inside a batched weight-quantization launch.  Descriptors of one
// launch travel by value in the kernel arguments (no device table, no allocation).
struct WeightDescDev {
  const void* w;
  void* q;
  float* s;
  int64_t ld_w;
  int64_t ld_q;
  int32_t first_block;  // first block id of this tensor within the launch
  int32_t kblocks;      // k / 128
  int32_t first_quad;   // first workgroup id of this tensor in a launch of 4-block workgroups
  int32_t kquads;       // ceil(kblocks / 4)
};

constexpr int kWeightChunk = 64;  // descriptors per launch (3.5 KB of kernel arguments)

struct WeightChunk {
  int32_t count;
  WeightDescDev d[kWeightChunk];
};
static_assert(sizeof(WeightChunk) <= 4096, "kernel arguments are limited to 4 KB");

// blocks: 128x128 blocks of the chunk; quads: workgroups of the chunk when each takes four
// blocks of a block row (the sum of n/128 * kquads)
hipError_t launch_quant_weight_chunk(const WeightChunk& chunk, int64_t blocks, int64_t quads, bool pow2,
                                     hipStream_t stream);

hipError_t launch_quant_act(const void* x, int64_t m, int64_t k, int64_t ld_x, void* q, int64_t ld_q,
                            float* s, int64_t ld_s, bool pow2, hipStream_t stream);

hipError_t launch_kv_quant(const void* k, int64_t ld_k, const void* v, int64_t ld_v, int64_t tokens,
                           int32_t heads, const int64_t* slots, void* k_cache, void* v_cache,
                           float* k_scale, float* v_scale, float range, bool recalibrate,
                           hipStream_t stream);

// pow2: the scales are powers of two (UE8M0 variant) and are applied by the matrix core
hipError_t launch_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                       int64_t ld_b, const float* b_s, void* y, int64_t ld_y, int64_t m, int64_t n,
                       int64_t k, bool pow2, hipStream_t stream);

// few tokens (m <= 64) with bf16 activations quantized inside the GEMM
hipError_t launch_gemm_bf16act(const void* x, int64_t ld_x, const void* b, int64_t ld_b, const float* b_s, void* y,
                               int64_t ld_y, int64_t m, int64_t n, int64_t k, bool pow2, hipStream_t stream);
hipError_t launch_grouped_swiglu(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as, const void* b,
                                 const float* b_s, const int32_t* offsets, int32_t groups, int64_t total_m,
                                 int64_t half, int64_t k, void* q, int64_t ld_q, float* s, int64_t ld_s,
                                 const int32_t* row_token, int64_t token_rows, bool pow2, hipStream_t stream);
hipError_t launch_grouped_gemm(const void* a, int64_t ld_a, const float* a_s, int64_t ld_as,
                               const void* b, const float* b_s, const int32_t* offsets, int32_t groups,
                               int64_t total_m, void* y, int64_t ld_y, int64_t n, int64_t k, bool pow2,
                               hipStream_t stream);

hipError_t launch_moe_dispatch(const void* xq, int64_t ld_xq, const float* xs, int64_t ld_xs, const int16_t* ids,
                               int64_t tokens, int32_t topk, int32_t experts, int64_t k, void* aq, int64_t ld_aq,
                               float* as, int64_t ld_as, int32_t* offsets, int32_t* row_of, hipStream_t stream);
hipError_t launch_moe_route(const int16_t* ids, int64_t tokens, int32_t topk, int32_t experts, int32_t* offsets,
                            int32_t* row_of, int32_t* row_token, hipStream_t stream);
hipError_t launch_swiglu_quant(const void* h, int64_t m, int64_t n, int64_t ld_h, void* q, int64_t ld_q, float* s,
                               int64_t ld_s, bool pow2, hipStream_t stream);
hipError_t launch_moe_combine(const void* y, int64_t ld_y, const int32_t* row_of, const float* w, int64_t tokens,
                              int32_t topk, int64_t hidden, void* out, int64_t ld_out, hipStream_t stream);
hipError_t launch_decode_attention(const void* q, int64_t ld_q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int64_t ld_bt, const int32_t* seq_lens, int32_t seqs,
                                   int32_t hq, int32_t hkv, int32_t page_size, float* q_scale, const float* k_scale,
                                   const float* v_scale, float sm_scale, float range, bool recalibrate, void* out,
                                   int64_t ld_out, hipStream_t stream);
}  // namespace fp8q

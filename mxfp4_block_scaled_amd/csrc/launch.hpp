// Internal launchers (host side). Each returns 0 on success, -1 if a launch failed.
// Arguments are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mxf {

int launch_quantize_act(const void* x, bool f32_in, int64_t rows, int64_t K, bool fp4, uint8_t* q,
                        uint8_t* q_scale, hipStream_t stream);

// routing: returns 1 if the sizes are outside what the kernels handle (nothing launched)
int route_permute_supported(int64_t T, int E, int topk);
// quantisation and routing in one launch for T <= 64 tokens and E <= 256 experts (route.hip)
int quantize_route_supported(int64_t T, int E);
int launch_quantize_route(const void* x, bool f32_in, int64_t H, bool fp4, uint8_t* q, uint8_t* q_scale,
                          const float* logits, int64_t T, int E, int topk, int32_t* topk_ids, float* gates,
                          int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row, hipStream_t stream);
int launch_route_permute(const float* logits, int64_t T, int E, int topk, int32_t* topk_ids,
                         float* gates, int32_t* expert_offsets, int32_t* sorted_pair,
                         int32_t* pair_row, hipStream_t stream);

int launch_combine(const void* y, bool y_bf16, const float* gates, const int32_t* pair_row,
                   int64_t T, int topk, int64_t H, void* out, bool out_bf16, hipStream_t stream);

// number of K slices the dense GEMM splits into (1: none); with more than one it
// needs dense_ksplit * M * N fp32 of partial sums
int dense_ksplit(int64_t M, int64_t N, int64_t K);
// the tiled kernels (many rows per weight matrix) address an activation matrix of
// `rows` rows and one [N][K/2] weight matrix with 32-bit byte offsets
bool tile_offsets_fit(int64_t rows, int64_t K, int64_t N, bool act_fp4);

// dense C[M][N] (fp32) = A_hat (already quantised, [M][K] codes + scales) x W_hat^T;
// partials: dense_ksplit(M, N, K) * M * N fp32 of scratch when that is above 1
int launch_dense_gemm(const uint8_t* qa, const uint8_t* qa_scale, bool act_fp4, int64_t M, int64_t N,
                      int64_t K, const uint8_t* w, const uint8_t* w_scale, float* c, float* partials,
                      hipStream_t stream);

// dense GEMMs of at most kDenseQRows rows take the bf16 activations straight into the
// weight-streaming kernel, which quantises them in registers (the codes never leave the
// compute unit): one launch when dense_q_ksplit is 1, else K slices of dense_ksplit
// and their fixed-order sum, needing dense_q_ksplit * M * N fp32 of partial sums
constexpr int64_t kDenseQRows = 16;
int dense_q_ksplit(int64_t M, int64_t N, int64_t K);
int launch_dense_q_gemm(const uint16_t* a, bool act_fp4, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                        const uint8_t* w_scale, float* c, float* partials, hipStream_t stream);

// FP4 weights x bf16 activations (gemm_w4a16.hip): K slices of 4 super-steps for narrow N
// (w4a16_ksplit > 1 needs w4a16_ksplit * min(M, 64) * N fp32 of partial sums)
int w4a16_ksplit(int64_t M, int64_t N, int64_t K);
int launch_w4a16_gemm(bool nvfp4, const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                      const uint8_t* ws, float* c, float* partials, hipStream_t stream);

// the lookup-table route (gemm_q8.hip): Q8 activations and int8-expanded MXFP4 weights
int launch_q8_quantize(const uint16_t* x, int64_t rows, int64_t K, int8_t* q, uint16_t* d, hipStream_t stream);
int launch_q8_gemm(const int8_t* q, const uint16_t* d, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                   const uint8_t* ws, float* c, float* partials, hipStream_t stream);

int launch_grouped_gemm(const uint8_t* q, const uint8_t* q_scale, bool act_fp4, int64_t T, int topk,
                        int64_t H, int64_t I, int E, const int32_t* expert_offsets,
                        const int32_t* sorted_pair, const uint8_t* w1, const uint8_t* w1_scale,
                        const uint8_t* w2, const uint8_t* w2_scale, uint8_t* h, uint8_t* h_scale,
                        void* y, bool y_bf16, hipStream_t stream);

// decode-sized batches (T <= 64): FC1 through the weight-streaming kernel, then FC2 fused
// with the gate-weighted combine (fc2_combine.hip); -1 when T > 64
int launch_grouped_gemm_combine(const uint8_t* q, const uint8_t* q_scale, bool act_fp4, int64_t T, int topk,
                                int64_t H, int64_t I, int E, const int32_t* expert_offsets,
                                const int32_t* sorted_pair, const int32_t* topk_ids, const int32_t* pair_row,
                                const float* gates, const uint8_t* w1,
                                const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale, uint8_t* h,
                                uint8_t* h_scale, void* out, bool out_bf16, hipStream_t stream);
int launch_fc2_combine(const uint8_t* h, const uint8_t* h_scale, bool act_fp4, int64_t T, int topk, int64_t H,
                       int64_t I, const int32_t* topk_ids, const int32_t* pair_row, const float* gates,
                       const uint8_t* w2, const uint8_t* w2_scale, void* out, bool out_bf16, hipStream_t stream);

}  // namespace mxf

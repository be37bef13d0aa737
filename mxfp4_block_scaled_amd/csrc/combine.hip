// Gate-weighted unpermute-combine (the "combine" half of MoE dispatch/combine,
// page "Domestic GPUs are awesome! Moore thread full-link adaptation DeepSeek-V4"):
//   out[t][n] = sum_{j=0..topk-1} gates[t][j] * y[pair_row[t*topk+j]][n]
// fp32 fused multiply-add in slot order j = 0..topk-1, then bf16 (RNE) or fp32.
// One thread owns 8 consecutive columns of one token: 16 B (bf16) / 32 B (fp32)
// per y row read, 16 B / 32 B written. HBM-bound.
#include "launch.hpp"

namespace mxf {

// y is read exactly once and out written once, each as whole lines (a wave covers
// 1 KB of one row): both go through non-temporal loads / stores, which measured
// faster for this single pass than cached accesses.
typedef unsigned int u4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

template <bool kYBF16>
__device__ __forceinline__ void load8(const void* y, int64_t off, float (&v)[8]) {
  if (kYBF16) {
    const u4v w = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(static_cast<const uint16_t*>(y) + off));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  } else {
    const f4v* p = reinterpret_cast<const f4v*>(static_cast<const float*>(y) + off);
    const f4v a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = a[j];
      v[4 + j] = b[j];
    }
  }
}

// KT > 0: topk is a compile-time constant and the KT gathered rows of a thread are
// all in flight at once (indices and gates first, then the rows, then the sum in
// slot order); KT == 0: any topk, one row at a time.
template <bool kYBF16, bool kOutBF16, int KT>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ pair_row,
                                                      int64_t T, int topk, int64_t H,
                                                      void* __restrict__ out) {
  const int64_t per_row = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row;
  const int64_t col = (idx - t * per_row) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  if constexpr (KT > 0) {
    int64_t r[KT];
    float gv[KT], v[KT][8];
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      r[j] = pair_row[t * KT + j];
      gv[j] = gates[t * KT + j];
    }
#pragma unroll
    for (int j = 0; j < KT; ++j) load8<kYBF16>(y, r[j] * H + col, v[j]);
#pragma unroll
    for (int j = 0; j < KT; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(gv[j], v[j][i], acc[i]);
  } else {
    for (int j = 0; j < topk; ++j) {
      const float g = gates[t * topk + j];
      const int64_t r = pair_row[t * topk + j];
      float v[8];
      load8<kYBF16>(y, r * H + col, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(g, v[i], acc[i]);
    }
  }
  if (kOutBF16) {
    u4v w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = bf16_round(acc[2 * i]) | (bf16_round(acc[2 * i + 1]) << 16);
    __builtin_nontemporal_store(w, reinterpret_cast<u4v*>(static_cast<uint16_t*>(out) + t * H + col));
  } else {
    f4v* p = reinterpret_cast<f4v*>(static_cast<float*>(out) + t * H + col);
    __builtin_nontemporal_store(f4v{acc[0], acc[1], acc[2], acc[3]}, p);
    __builtin_nontemporal_store(f4v{acc[4], acc[5], acc[6], acc[7]}, p + 1);
  }
}

int launch_combine(const void* y, bool y_bf16, const float* gates, const int32_t* pair_row,
                   int64_t T, int topk, int64_t H, void* out, bool out_bf16, hipStream_t stream) {
  const int64_t n = T * (H / 8);
  if (n == 0) return 0;
  dim3 grid((unsigned)cdiv(n, 256)), block(256);
  if (y_bf16) {
    if (out_bf16 && topk == 6) combine_kernel<true, true, 6><<<grid, block, 0, stream>>>(y, gates, pair_row, T, topk, H, out);
    else if (out_bf16) combine_kernel<true, true, 0><<<grid, block, 0, stream>>>(y, gates, pair_row, T, topk, H, out);
    else if (topk == 6) combine_kernel<true, false, 6><<<grid, block, 0, stream>>>(y, gates, pair_row, T, topk, H, out);
    else combine_kernel<true, false, 0><<<grid, block, 0, stream>>>(y, gates, pair_row, T, topk, H, out);
  } else {
    if (out_bf16) combine_kernel<false, true, 0><<<grid, block, 0, stream>>>(y, gates, pair_row, T, topk, H, out);
    else combine_kernel<false, false, 0><<<grid, block, 0, stream>>>(y, gates, pair_row, T, topk, H, out);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

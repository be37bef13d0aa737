// Activation quantisation to MXFP8 (E4M3) or MXFP4 (E2M1) with UE8M0 block scales.
// One thread owns one 32-element block: 64 B (bf16) or 128 B (fp32) in,
// 32 B or 16 B of codes + 1 scale byte out. HBM-bound; the rule is in mx_codec.hpp.
#include "launch.hpp"
#include "mx_codec.hpp"

namespace mxf {

template <bool kF32In, bool kFP4>
__global__ void __launch_bounds__(256) quantize_act_kernel(const void* __restrict__ x, int64_t nblocks,
                                                           uint8_t* __restrict__ q,
                                                           uint8_t* __restrict__ q_scale) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b < nblocks) quantize_act_block<kF32In, kFP4>(x, b, q, q_scale);
}

int launch_quantize_act(const void* x, bool f32_in, int64_t rows, int64_t K, bool fp4, uint8_t* q,
                        uint8_t* q_scale, hipStream_t stream) {
  const int64_t nblocks = rows * (K / 32);
  if (nblocks == 0) return 0;
  dim3 grid((unsigned)cdiv(nblocks, 256)), block(256);
  if (f32_in) {
    if (fp4)
      quantize_act_kernel<true, true><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale);
    else
      quantize_act_kernel<true, false><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale);
  } else {
    if (fp4)
      quantize_act_kernel<false, true><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale);
    else
      quantize_act_kernel<false, false><<<grid, block, 0, stream>>>(x, nblocks, q, q_scale);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

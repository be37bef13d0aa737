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
  if (b >= nblocks) return;
  float v[32];
  if (kF32In) {
    const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + b * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4 f = src[i];
      v[4 * i + 0] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + b * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 w = src[i];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j + 0] = __uint_as_float(ws[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
      }
    }
  }
  uint32_t out[8];
  const uint32_t byte = quantize_block32<kFP4>(v, out);
  if (kFP4) {
    *reinterpret_cast<uint4*>(q + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
  } else {
    uint4* dst = reinterpret_cast<uint4*>(q + b * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  }
  q_scale[b] = (uint8_t)byte;
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

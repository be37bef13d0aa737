// Bit-exact MX block quantisation on the device (integer arithmetic on fp32 bits).
//
// One 32-element block follows the OCP Microscaling (MX) v1.0 conversion with
// the element formats the pages name: E2M1 (1 sign / 2 exponent / 1 mantissa
// bit, page "DGX Spark 原生 FP4 矩阵指令" section 一, with the UE8M0 block scale
// of the same section) and E4M3 (4 exponent / 3 mantissa bits, page
// "企业官网建设流程全解析" section 一, OCP "FN" variant: no infinities, max 448).
//   scale byte  = max(0, biased exponent of amax - emax)   (emax 8 / 2)
//               = clamp(floor(log2 amax) - emax + 127, 0, 254) for finite amax
//   element     = round-to-nearest-even of v * 2^(127 - byte) on the element
//                 grid (subnormals included), saturating at the largest normal,
//                 sign bit copied from v (so -0 and negative underflow give -0).
// The multiply by a power of two is exact unless the product falls below
// 2^-126, where every element code is 0 anyway.
#pragma once

#include "common.hpp"

namespace mxf {

constexpr uint32_t kEmaxE4M3 = 8;
constexpr uint32_t kEmaxE2M1 = 2;

__device__ __forceinline__ uint32_t scale_byte_from_amax_bits(uint32_t amax_bits, uint32_t emax) {
  uint32_t e = (amax_bits >> 23) & 0xFFu;
  return e > emax ? e - emax : 0u;
}

// 2^(127 - byte) as fp32; valid for byte in [0, 253] (the quantiser produces <= 246)
__device__ __forceinline__ float inv_scale_from_byte(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// |t| -> 7-bit E4M3 magnitude code (0x00 .. 0x7E). Every case is computed and the
// right one selected, so a wave runs no branches per element.
__device__ __forceinline__ uint32_t e4m3_mag_code(float a) {
  // below 2^-6: subnormal grid m * 2^-9, m = 0..8 (8 = 2^-6)
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(a, 0.015625f) * 512.0f);
  const uint32_t u = __float_as_uint(a);
  const uint32_t nrm = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);  // (exp << 3 | m3), rounded
  return a >= 448.0f ? 0x7Eu : (a < 0.015625f ? sub : nrm);
}

// |t| -> 3-bit E2M1 magnitude code (0 .. 7), branch-free like e4m3_mag_code
__device__ __forceinline__ uint32_t e2m1_mag_code(float a) {
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(a, 1.0f) * 2.0f);  // 0, 0.5, 1.0 below 1
  const uint32_t u = __float_as_uint(a);
  const uint32_t r = (u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22;  // (exp << 1 | m1), rounded
  const uint32_t nrm = min(r - ((127u - 1u) << 1), 7u);
  return a >= 6.0f ? 7u : (a < 1.0f ? sub : nrm);
}

__device__ __forceinline__ uint32_t e4m3_code(float v, float inv_scale) {
  uint32_t s = (__float_as_uint(v) >> 24) & 0x80u;
  return s | e4m3_mag_code(fabsf(v) * inv_scale);
}

__device__ __forceinline__ uint32_t e2m1_code(float v, float inv_scale) {
  uint32_t s = (__float_as_uint(v) >> 28) & 0x8u;
  return s | e2m1_mag_code(fabsf(v) * inv_scale);
}

// Quantise 32 fp32 values of one block held by one thread.
// E4M3: out32 receives 32 bytes (8 words, little-endian element order).
// E2M1: out32 receives 16 bytes (4 words), element 2n in the low nibble of byte n.
template <bool kFP4>
__device__ __forceinline__ uint32_t quantize_block32(const float (&v)[32], uint32_t (&out)[8]) {
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = max(amax, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  const uint32_t byte = scale_byte_from_amax_bits(amax, kFP4 ? kEmaxE2M1 : kEmaxE4M3);
  const float inv = inv_scale_from_byte(byte);
  if (kFP4) {
#if defined(__HIP_DEVICE_COMPILE__)
    // gfx950's scaled E2M1 conversion (v / scale, round to nearest even on the E2M1
    // grid, saturating, sign kept) gives exactly e2m1_code(v, 1 / scale): checked on
    // the GPU for every finite bf16 pattern, a million random fp32 values and the
    // grid midpoints with their neighbours, scale bytes 117..137. Blocks with a scale
    // byte below 64 are lifted by 2^64 (values and scale alike, exact) so that the
    // scale operand and the elements stay normal fp32 numbers.
    const bool lift = byte < 64u;
    const float mul = lift ? 18446744073709551616.0f : 1.0f;
    const float sc = __uint_as_float((byte + (lift ? 64u : 0u)) << 23);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* x = &v[w * 8];
      uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x[0] * mul, x[1] * mul, sc, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x[2] * mul, x[3] * mul, sc, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x[4] * mul, x[5] * mul, sc, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, x[6] * mul, x[7] * mul, sc, 3);
      out[w] = word;
    }
    (void)inv;
#else
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 8; ++n) word |= e2m1_code(v[w * 8 + n], inv) << (4 * n);
      out[w] = word;
    }
#endif
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int n = 0; n < 4; ++n) word |= e4m3_code(v[w * 4 + n], inv) << (8 * n);
      out[w] = word;
    }
  }
  return byte;
}

// One 32-element block b of the activations (bf16 or fp32): codes and scale byte.
template <bool kF32In, bool kFP4>
__device__ __forceinline__ void quantize_act_block(const void* __restrict__ x, int64_t b, uint8_t* __restrict__ q,
                                                   uint8_t* __restrict__ q_scale) {
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

}  // namespace mxf

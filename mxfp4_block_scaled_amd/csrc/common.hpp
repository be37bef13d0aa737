// Shared device helpers for the gfx950 (CDNA4) kernels of the MXFP4 expert path.
//
// Scaled-MFMA operand layout (measured on gfx950 with an in-bounds probe and
// relied on by every GEMM kernel here). For
//   v_mfma_scale_f32_16x16x128_f8f6f4  (R = 16 rows, G = 4 lane groups) and
//   v_mfma_scale_f32_32x32x64_f8f6f4   (R = 32 rows, G = 2 lane groups)
// with operands A (rows i) and B (rows j), both K-contiguous ("nt"):
//   C[i][j] += sum_k A[i][k] * sa(i, k/32) * B[j][k] * sb(j, k/32)
// * lane l supplies row l % R of its operand;
// * FP4 (E2M1) operand: lane l holds the whole 32-element block g = l / R in
//   its first 16 bytes, element 2n in the low nibble of byte n;
// * FP8 (E4M3) operand: lane l holds k in [16g, 16g+16) in bytes 0..15 and
//   k in [16G + 16g, 16G + 16g + 16) in bytes 16..31;
// * scales: lane l supplies the E8M0 byte (op_sel picks one byte of a 32-bit
//   register) of row l % R, block l / R - regardless of the element format;
// * 16x16 result: lane l holds C[4(l/16) + v][l % 16], v = 0..3;
//   32x32 result: lane l holds C[8(v/4) + 4(l/32) + v%4][l % 32], v = 0..15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxf {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// format selectors of the scaled MFMA (cbsz / blgp fields)
constexpr int kFmtFP8 = 0;  // E4M3
constexpr int kFmtFP4 = 4;  // E2M1

// OPS selects which byte of the two 32-bit scale registers is used (same for A and B)
template <int FA, int FB, int OPS>
__device__ __forceinline__ v4f mfma16x16x128(const v8i& a, const v8i& b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, OPS, sa, OPS, sb);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Workgroup barrier for LDS hand-offs that leaves global loads in flight.
// __syncthreads() makes the compiler drain every outstanding memory counter
// (vmcnt included) first, which would cancel register prefetches issued for
// later stages. Here only this wave's LDS operations are waited for (lgkmcnt),
// which is what makes its LDS writes visible to the other waves after the
// barrier; the asm's memory clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float wave_max16(float v) {
  // max over the 16 lanes that share l / 16 (butterfly inside each 16-lane row)
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}

__device__ __forceinline__ uint32_t bf16_round(float f) {
  // fp32 -> bf16 bits, round to nearest even (inputs here are finite)
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace mxf

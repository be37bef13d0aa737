// Achievable-rate probes: a streaming read of HBM, a register-only loop of
// block-scaled 32x32x64 MFMAs, and the HBM -> LDS copy path of the prefill GEMMs
// on its own. They measure what the chip sustains for the bounds of the expert
// path (its weight-streaming decode kernels, its prefill GEMMs' matrix cores and
// their operand copies), so that the measured kernels can be reported against
// those rates as well as against the datasheet peaks. Contracts in
// include/mxf_ceilings.h.
#include "mxf_ceilings.h"

#include <hip/hip_runtime.h>

namespace {

typedef int v4i_c __attribute__((ext_vector_type(4)));
typedef int v8i_c __attribute__((ext_vector_type(8)));
typedef float v16f_c __attribute__((ext_vector_type(16)));

// operand format codes of the f8f6f4 instructions
constexpr int kCodeE4M3 = 0, kCodeE2M1 = 4;
constexpr int kReadGroups = 4096;

// Each wave loads one operand set (2 A and 4 B fragments, 8 words per lane each)
// and then runs `iters` rounds of the 8 independent products A_i x B_j, as the
// wide GEMM kernel's inner step does. E2M1 operands use the low 4 words of a
// fragment (16 bytes per lane); E4M3 A uses all 8, with the lowest bit of every
// byte cleared so that no byte is the NaN code. Registers are held to two waves
// per SIMD (the launch puts two workgroups on each compute unit).
template <int kFmtA>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) ceiling_mfma_kernel(
    const int* __restrict__ ops, int scale, int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int set = (int)((blockIdx.x * 4u + (threadIdx.x >> 6)) & 63u);
  const int* src = ops + (size_t)set * (6 * 64 * 8);
  v8i_c a[2], b[4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int w = src[(f * 64 + lane) * 8 + i];
      a[f][i] = kFmtA == kCodeE4M3 ? (w & (int)0xFEFEFEFE) : (i < 4 ? w : 0);
    }
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) b[f][i] = i < 4 ? src[((2 + f) * 64 + lane) * 8 + i] : 0;
  v16f_c acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f_c{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], kFmtA, kCodeE2M1, 0,
                                                                    scale, 0, scale);
  }
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) t += acc[i][j][v];
  if (threadIdx.x == 0) sink[blockIdx.x] = t;
}

// Grid-stride streaming read: a wave's load instruction covers 1 KB contiguous
// (eight whole 128-byte lines), non-temporal (every line is read once).
__global__ void __launch_bounds__(256) ceiling_read_kernel(const v4i_c* __restrict__ p, int64_t n16,
                                                           int* __restrict__ xor_out) {
  __shared__ int red[4];
  const int64_t stride = (int64_t)gridDim.x * 256;
  int acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const v4i_c v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) acc ^= __shfl_xor(acc, d);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) atomicXor(xor_out, red[0] ^ red[1] ^ red[2] ^ red[3]);
}

// LDS-fill probe (contract in mxf_ceilings.h). Copy q of wave w at stage st moves 1 KB:
// q < 4 from the activation region, q >= 4 from the weight region, piece (4 w + q % 4)
// of the region's 32 KB stage chunk, landing at (q < 4 ? 0 : 32 KB) + piece * 1 KB of
// the stage's half. Raw buffer resources over one region each (64-bit base, 32-bit
// offsets below MXF_CEILING_COPY_REGION): an out-of-range lane would read zero.
typedef __amdgpu_buffer_rsrc_t rsrc_c;
__device__ __forceinline__ rsrc_c region_rsrc(const uint8_t* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, MXF_CEILING_COPY_REGION, 0x00020000);
}
__global__ void __launch_bounds__(512) ceiling_lds_copy_kernel(const uint8_t* __restrict__ buf, int pattern, int groups,
                                                               uint32_t* __restrict__ sum_out) {
  __shared__ __attribute__((aligned(16))) uint8_t half[2][65536];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int b = blockIdx.x, x = b & 7, j = b >> 3, k = j >> 5, i = j & 31;
  int64_t ra, rb;
  if (pattern == 0) {
    ra = b;
    rb = (int64_t)groups + b;
  } else {
    ra = (int64_t)(8 * k + x) * 2 + (i & 1);
    rb = (int64_t)groups / 16 + (int64_t)(8 * k + x) * 16 + (i >> 1);
  }
  const rsrc_c sa = region_rsrc(buf + ra * MXF_CEILING_COPY_REGION);
  const rsrc_c sb = region_rsrc(buf + rb * MXF_CEILING_COPY_REGION);
  auto issue = [&](int st) {
    uint8_t* d = half[st & 1];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int piece = 4 * wave + (q & 3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 4 ? sa : sb,
                                               (__attribute__((address_space(3))) void*)(d + (q < 4 ? 0 : 32768) + piece * 1024),
                                               16, 16 * lane + piece * 1024, st * 32768, 0, 0);
    }
  };
  uint32_t sum = 0;
  issue(0);
  for (int st = 0; st < MXF_CEILING_COPY_STAGES; ++st) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of stage st have landed
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (st + 1 < MXF_CEILING_COPY_STAGES) issue(st + 1);
    const uint8_t* d = half[st & 1];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const v4i_c v = *reinterpret_cast<const v4i_c*>(d + (8 * wave + q) * 1024 + 16 * lane);
      sum += (uint32_t)v[0] + (uint32_t)v[1] + (uint32_t)v[2] + (uint32_t)v[3];
    }
  }
#pragma unroll
  for (int dd = 32; dd > 0; dd >>= 1) sum += (uint32_t)__shfl_xor((int)sum, dd);
  if (lane == 0) atomicAdd(sum_out, sum);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int64_t mxf_ceiling_mfma_flops(int iters) {
  return iters <= 0 ? 0 : (int64_t)MXF_CEILING_MFMA_GROUPS * 4 * (int64_t)iters * 8 * 131072;
}

int mxf_ceiling_mfma(int act_fmt, const int32_t* operands, int64_t operand_words, int scale, int iters,
                     float* sink, mxf_stream stream) {
  if (act_fmt != MXF_E4M3 && act_fmt != MXF_E2M1) return MXF_ERR_FORMAT;
  if (iters < 1 || iters > 1000000 || operand_words < MXF_CEILING_MFMA_WORDS || scale < 0 || scale > 254)
    return MXF_ERR_SHAPE;
  if (!operands || !sink) return MXF_ERR_NULL;
  if (!aligned16(operands) || !aligned16(sink)) return MXF_ERR_ALIGN;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (act_fmt == MXF_E2M1)
    ceiling_mfma_kernel<kCodeE2M1><<<MXF_CEILING_MFMA_GROUPS, 256, 0, s>>>(operands, scale, iters, sink);
  else
    ceiling_mfma_kernel<kCodeE4M3><<<MXF_CEILING_MFMA_GROUPS, 256, 0, s>>>(operands, scale, iters, sink);
  return hipGetLastError() == hipSuccess ? MXF_OK : MXF_ERR_LAUNCH;
}

int mxf_ceiling_read(const void* buf, int64_t bytes, int32_t* xor_out, mxf_stream stream) {
  if (bytes < 0 || bytes % 16 != 0) return MXF_ERR_SHAPE;
  if (bytes == 0) return MXF_OK;
  if (!buf || !xor_out) return MXF_ERR_NULL;
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(xor_out) & 3u) != 0) return MXF_ERR_ALIGN;
  const int64_t n16 = bytes / 16;
  const int64_t need = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(need < kReadGroups ? need : kReadGroups);
  ceiling_read_kernel<<<grid, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const v4i_c*>(buf), n16, xor_out);
  return hipGetLastError() == hipSuccess ? MXF_OK : MXF_ERR_LAUNCH;
}

int64_t mxf_ceiling_lds_copy_bytes(int pattern, int groups) {
  if (groups <= 0 || groups % 256 != 0 || groups > 65536) return 0;
  if (pattern == 0) return (int64_t)2 * groups * MXF_CEILING_COPY_REGION;
  if (pattern == 1) return (int64_t)(groups / 16 + groups / 2) * MXF_CEILING_COPY_REGION;
  return 0;
}

int mxf_ceiling_lds_copy(const void* buf, int64_t bytes, int pattern, int groups, uint32_t* sum_out,
                         mxf_stream stream) {
  const int64_t need = mxf_ceiling_lds_copy_bytes(pattern, groups);
  if (need == 0 || bytes < need) return MXF_ERR_SHAPE;
  if (!buf || !sum_out) return MXF_ERR_NULL;
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(sum_out) & 3u) != 0) return MXF_ERR_ALIGN;
  ceiling_lds_copy_kernel<<<(unsigned)groups, 512, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(buf), pattern, groups, sum_out);
  return hipGetLastError() == hipSuccess ? MXF_OK : MXF_ERR_LAUNCH;
}

}  // extern "C"

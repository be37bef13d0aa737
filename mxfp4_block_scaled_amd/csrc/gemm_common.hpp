// Shared pieces of the MXFP4 GEMM kernels (weight-streaming and LDS-ring):
// the argument block, the expert/work-unit lookup over expert_offsets, the
// 32x32x64 scaled MFMA, the per-32 requantisation of one staged row block, and
// the HBM -> LDS copy and wait primitives.
//
// The weights stay E2M1 + UE8M0 all the way into the matrix instruction - no
// dequantisation to a 16-bit type (page "DGX Spark 原生 FP4 矩阵指令" sections 一
// and 二). Activations are E4M3 (FP8 x FP4) or E2M1 (FP4 x FP4); products are
// exact and accumulate in fp32. FC1's epilogue fuses SwiGLU and the
// requantisation of h per 32 along I (page "Domestic GPUs are awesome! ...
// DeepSeek-V4": "SwiGLU + FP8 quant").
#pragma once

#include <type_traits>

#include "launch.hpp"
#include "mx_codec.hpp"

namespace mxf {

enum { kModeFC1 = 0, kModeFC2 = 1, kModeDense = 2 };

struct GemmArgs {
  const uint8_t* act;        // FC1: q [T][K(/2)], FC2: h [R][K(/2)], dense: qa [M][K(/2)]
  const uint8_t* act_scale;  // [.][K/32]
  const uint8_t* w;          // [E][N][K/2]
  const uint8_t* w_scale;    // [E][N][K/32]
  const int32_t* offsets;    // [E+1] (FC1/FC2)
  const int32_t* sorted_pair;
  uint8_t* h;                // FC1 out [R][I(/2)]
  uint8_t* h_scale;          // FC1 out [R][I/32]
  void* out;                 // FC2: y [R][N]; dense: c [M][N]
  int64_t K, N, I, M;
  int64_t act_rows;  // rows of act / act_scale (FC1: T, FC2: T * topk, dense: M)
  int topk, E;
  int ntiles;  // tile kernel: weight-row tiles per expert (1-D grid: block = m_unit * ntiles + n_tile)
  int kchunk;  // dense weight-streaming kernel: 512-k super-steps per grid.y slice (0: the whole K)
  int ngroup;  // wide kernel, grouped GEMMs: consecutive n-tiles per workgroup (ntiles % ngroup == 0; 0: one)
  int split;   // grouped GEMMs: experts with 1..split rows run in the streaming kernel, the
               // others in the tiled kernels (0: every non-empty expert in the launched kernel)
};

// ---------------------------------------------------------------------------------
// Which expert does work unit u belong to? units(e) = (count_e > 0) when BM == 0 (the
// streaming kernel), else ceil(count_e / BM); with split > 0 the streaming kernel
// counts only experts of at most split rows and the tiled kernels only the others.
// Called by a whole wave; results are wave-uniform.
template <int BM>
__device__ __forceinline__ int units_of(int c, int split) {
  if constexpr (BM == 0) return c > 0 && (split == 0 || c <= split) ? 1 : 0;
  else return split > 0 && c <= split ? 0 : (c + BM - 1) / BM;
}

template <int BM>
__device__ __forceinline__ void find_unit(const int32_t* __restrict__ off, int E, int split, int u, int& e_out,
                                          int& loc_out) {
  const int lane = threadIdx.x & 63;
  const int C = (E + 63) >> 6;
  const int first = lane * C;
  int units = 0;
  for (int i = 0; i < C; ++i) {
    const int e = first + i;
    if (e < E) {
      const int c = off[e + 1] - off[e];
      units += units_of<BM>(c, split);
    }
  }
  int incl = units;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int excl = incl - units;
  const bool mine = u >= excl && u < incl;
  const unsigned long long m = __ballot(mine);
  if (m == 0) {
    e_out = -1;
    loc_out = 0;
    return;
  }
  const int src = __ffsll((long long)m) - 1;
  int ee = -1, loc = 0;
  if (mine) {
    int acc = excl;
    for (int i = 0; i < C; ++i) {
      const int e = first + i;
      if (e < E) {
        const int c = off[e + 1] - off[e];
        const int n = units_of<BM>(c, split);
        if (u < acc + n) {
          ee = e;
          loc = u - acc;
          break;
        }
        acc += n;
      }
    }
  }
  e_out = __shfl(ee, src);
  loc_out = __shfl(loc, src);
}

// the value of lane l ^ 32 (a swap of the wave's halves): gfx950's
// v_permlane32_swap exchanges lanes 32..63 of its first operand with lanes 0..31 of
// its second, on the VALU (no LDS round trip); with both operands x, the first
// result holds x of lane l - 32 in the upper half, the second x of lane l + 32 in
// the lower half
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32u) ? r[0] : r[1];
#else
  return x;
#endif
}

// Work item of block j on XCD x for the grouped GEMMs (units of BM rows). Items run expert by expert;
// within an expert, n-tile by n-tile, and within an n-tile over the expert's units,
// so the workgroups resident on one XCD at a time cover one or two experts: each
// activation unit is shared by every n-tile there and each weight tile by the
// expert's units, and L2 holds both. The U * ntiles items are split into 8
// contiguous ranges, one per XCD (block b runs on XCD b % 8). Called by a whole
// wave; the results are wave-uniform. e_out < 0: no item for this block.
template <int BM>
__device__ __forceinline__ void grouped_work_item(const int32_t* __restrict__ off, int E, int split, int ntiles, int x,
                                                  int j, int& e_out, int& n_out, int& loc_out) {
  const int lane = threadIdx.x & 63;
  const int C = (E + 63) >> 6;
  const int first = lane * C;
  int units = 0;
  for (int i = 0; i < C; ++i) {
    const int e = first + i;
    if (e < E) units += units_of<BM>(off[e + 1] - off[e], split);
  }
  int incl = units;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int excl = incl - units;
  const int64_t total = (int64_t)__shfl(incl, 63) * ntiles;
  const int64_t w = x * total / 8 + j;
  e_out = -1;
  n_out = loc_out = 0;
  if (w >= (x + 1) * total / 8) return;
  const int p = (int)(w / ntiles);  // a unit of the wanted expert
  const bool mine = p >= excl && p < incl;
  const unsigned long long msk = __ballot(mine);
  if (msk == 0) return;
  const int src = __ffsll((long long)msk) - 1;
  int ee = -1, ue = 0, ke = 1;
  if (mine) {
    int acc = excl;
    for (int i = 0; i < C; ++i) {
      const int e = first + i;
      if (e < E) {
        const int n = units_of<BM>(off[e + 1] - off[e], split);
        if (p < acc + n) {
          ee = e;
          ue = acc;
          ke = n;
          break;
        }
        acc += n;
      }
    }
  }
  ee = __shfl(ee, src);
  ue = __shfl(ue, src);
  ke = __shfl(ke, src);
  const int64_t local = w - (int64_t)ue * ntiles;
  e_out = ee;
  n_out = (int)(local / ke);
  loc_out = (int)(local % ke);
}

// f(integral_constant<int, i>) for i = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// silu(g) * u with the hardware exponential and reciprocal (about 1 ulp each)
__device__ __forceinline__ float silu_mul(float g, float u) {
#if defined(__HIP_DEVICE_COMPILE__)
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
#else
  return g / (1.0f + __expf(-g)) * u;
#endif
}

// two fp32 values as packed bf16 bits (x in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t bf16x2_bits(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 r = __builtin_convertvector((f2){x, y}, b2);
  return __builtin_bit_cast(uint32_t, r);
}

template <bool kYBF16>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if (kYBF16)
    static_cast<uint16_t*>(out)[idx] = (uint16_t)bf16_round(x);
  else
    static_cast<float*>(out)[idx] = x;
}

template <int FA, int FB, int OPS>
__device__ __forceinline__ v16f mfma32x32x64(const v8i& a, const v8i& b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OPS, sa, OPS, sb);
}

// Quantise 32 consecutive fp32 values (one block of a row) held by one thread and
// store codes + scale byte; used by the staged FC1 epilogue.
template <bool kActFP4>
__device__ __forceinline__ void quantize_store32(const float* __restrict__ src, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scale) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    const float4 f = *reinterpret_cast<const float4*>(src + i);
    v[i] = f.x;
    v[i + 1] = f.y;
    v[i + 2] = f.z;
    v[i + 3] = f.w;
  }
  uint32_t out[8];
  const uint32_t byte = quantize_block32<kActFP4>(v, out);
  if (kActFP4) {
    *reinterpret_cast<uint4*>(codes) = make_uint4(out[0], out[1], out[2], out[3]);
  } else {
    reinterpret_cast<uint4*>(codes)[0] = make_uint4(out[0], out[1], out[2], out[3]);
    reinterpret_cast<uint4*>(codes)[1] = make_uint4(out[4], out[5], out[6], out[7]);
  }
  *scale = (uint8_t)byte;
}


// swizzle of the 16-byte chunk index inside a row (8 or 16 chunks per row)
template <int C>
__device__ __forceinline__ int swz(int r) {
  if constexpr (C == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return r & 15;
}

// HBM -> LDS copy of 16 (or 4) bytes per lane: lane l lands at lds + 16 l (4 l).
// The builtins below exist only for the device pass of the compiler.
__device__ __forceinline__ void dma16_to_lds(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}
__device__ __forceinline__ void dma4_to_lds(const void* src, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
#endif
}

// wait until at most N vector-memory loads of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
#endif
}

// Raw buffer resources (base, byte size): loads through them are range-checked
// by the hardware (out-of-range lanes read zero), and their HBM -> LDS form is a
// MUBUF instruction, which the compiler's wait-count tracking keeps apart from
// the plain register loads it can then wait for precisely.
#if defined(__HIP_DEVICE_COMPILE__)
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
#else
struct buf_rsrc {
  int w[4];
};
#endif
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  // dword 3 = 0x00020000: raw (untyped) 32-bit data format on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
#else
  (void)base;
  (void)bytes;
  return buf_rsrc{};
#endif
}
// 16 (or 4) bytes per lane from byte offset voff + soff to lds + 16 lane (4 lane)
__device__ __forceinline__ void buf_dma16(buf_rsrc r, void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, (int)soff, 0, 0);
#endif
}
__device__ __forceinline__ void buf_dma4(buf_rsrc r, void* lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, (int)voff, (int)soff, 0, 0);
#endif
}
__device__ __forceinline__ v4i buf_load16(buf_rsrc r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
#else
  return v4i{};
#endif
}
// non-temporal form (cache policy NT: lines read once, not kept in the caches)
__device__ __forceinline__ v4i buf_load16_nt(buf_rsrc r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2);
#else
  return v4i{};
#endif
}
__device__ __forceinline__ int buf_load4(buf_rsrc r, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
#else
  return 0;
#endif
}

// tile geometry of the LDS-ring kernels: 256 activation rows x 256 weight rows
namespace tile {
constexpr int BM = 256, BN = 256;
}  // namespace tile

// c[i] = sum over s < S of part[s * n + i], in the order s = 0 .. S-1 (n % 4 == 0)
void launch_reduce_partials(const float* part, int S, int64_t n, float* c, hipStream_t stream);

// kernel launchers (gemm_stream.hip, gemm_tile.hip); mode is kModeFC1 / kModeFC2 / kModeDense
void launch_stream_gemm(int mode, bool y_bf16, bool act_fp4, const GemmArgs& a, int mt, dim3 grid,
                        hipStream_t stream);
// dense GEMM with M <= 16 whose a.act holds the bf16 activations [M][K] (quantised in registers)
void launch_stream_q_gemm(bool act_fp4, const GemmArgs& a, dim3 grid, hipStream_t stream);
// rows: activation rows in all; groups: experts that may hold a partial unit (0 for dense)
// returns -1 (nothing launched) when an operand exceeds the tiled kernels' 32-bit offsets
int launch_tile_gemm(int mode, bool y_bf16, bool act_fp4, const GemmArgs& a, int64_t rows, int64_t groups,
                     hipStream_t stream);
void launch_wide_gemm(int mode, bool y_bf16, const GemmArgs& a, int64_t m_units, hipStream_t stream);
void launch_f8ring_gemm(int mode, bool y_bf16, const GemmArgs& a, int64_t m_units, hipStream_t stream);

}  // namespace mxf

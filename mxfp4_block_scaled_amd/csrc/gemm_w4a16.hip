// FP4-weight GEMM with bf16 activations ("W4A16"): C[M][N] (fp32) = A . W_hat^T with
// A in bf16 as given (no activation quantisation) and W_hat one of
//   MXFP4: E2M1 codes, one UE8M0 scale per 32 K-elements (the layer's weight format);
//   NVFP4: E2M1 codes, one UE4M3 scale per 16 K-elements (the block format behind the
//          pages' kind::mxf4nvf4 / scale_vec::4X instruction).
// gfx950's scaled matrix instructions take E8M0 scales per 32 elements, which can carry
// neither bf16 activations nor a per-16 non-power-of-two scale. So each lane decodes its
// weight codes with the block scale to bf16 in registers (code x scale is exact in bf16:
// an E2M1 value times a UE8M0 or UE4M3 scale has at most 5 significant bits) and runs
// the bf16 matrix instruction, accumulating in fp32. MXFP4 decodes with one scaled
// conversion per code pair (v_cvt_scalef32_pk_bf16_fp4); that conversion applies only
// the exponent of its scale operand (measured: UE4M3 scales through it came out wrong by
// their mantissa factor), so NVFP4 passes the scale's power of two through the
// conversion and multiplies by its mantissa factor 1 + m/8 in fp32. That is
// the fused dequantise + matmul of page "【DeepSeek V4】Triton FP4 优化实战" section
// 第二步, done in registers with no 16-bit weight copy in memory.
//
// Weight streaming as in gemm_stream.hip: a workgroup owns 64 weight rows, each wave a
// share of K; every weight byte is read once per launch as whole 128-byte lines
// (non-temporal) and passed through a per-wave LDS area into the matrix lane layout,
// so that lane (g, r16) holds the 16 bytes (32 codes) of row r16, 32-k block 4 s + g
// of a 512-k super-step at step s. Those 32 codes feed four 16x16x32 instructions: the
// K order inside a super-step is free as long as activations and weights share it, so
// instruction j of step s takes k = 32 (4 s + g) + 8 j + [0, 8) in lane group g - eight
// consecutive bf16 activations, a 16-byte load.
#include "gemm_common.hpp"

namespace mxf {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

namespace w16 {
constexpr int kStgStride = 1152;  // as in the streaming kernel: odd load instructions 128 B (mod 256) apart
constexpr int kStgBytes = 4 * kStgStride;
}  // namespace w16

struct W16Args {
  const uint16_t* a;  // [M][K] bf16
  const uint8_t* w;   // [N][K/2] E2M1 codes
  const uint8_t* ws;  // [N][K/32] UE8M0 (MXFP4) or [N][K/16] UE4M3 (NVFP4)
  float* out;         // [M][N], or [slices][M][N] partial sums when kchunk > 0
  int64_t M, N, K;
  int kchunk;         // 512-k super-steps per grid.y slice (0: the whole K)
};

// UE4M3 (OCP E4M3 with the sign bit clear) -> fp32, exact: exponent 0 is subnormal
// (m x 2^-9), otherwise 2^(e-7) (1 + m/8)
__device__ __forceinline__ float ue4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float sub = (float)m * 0.001953125f;
  const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// 2^(b - 127) as fp32 (b = 0: the subnormal 2^-127)
__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) { return __uint_as_float(b ? b << 23 : 0x00400000u); }

typedef float v2f __attribute__((ext_vector_type(2)));

// 8 E2M1 codes (one dword, element 2n in the low nibble of byte n) x a power-of-two
// scale -> 8 bf16 (the scaled conversion applies only the exponent of its fp32 scale)
__device__ __forceinline__ v8bf decode8(uint32_t codes, float scale) {
#if defined(__HIP_DEVICE_COMPILE__)
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#else
  (void)codes;
  (void)scale;
  return v8bf{};
#endif
}

// 8 E2M1 codes x a UE4M3 scale -> 8 bf16: the scale's power of two goes into the scaled
// conversion to fp32, its mantissa factor f = 1 + m/8 is multiplied in fp32 (both exact:
// a code times f has at most 5 significant bits), then each pair rounds to bf16 exactly
__device__ __forceinline__ v8bf decode8_nv(uint32_t codes, float scale) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t sb = __float_as_uint(scale);
  const float p = __uint_as_float(sb & 0x7F800000u);               // 2^floor(log2 scale); 0 for 0
  const float f = __uint_as_float((sb & 0x007FFFFFu) | 0x3F800000u);  // scale / p in [1, 2)
  const v2f x0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p, 0);
  const v2f x1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p, 1);
  const v2f x2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p, 2);
  const v2f x3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, p, 3);
  return v8bf{(__bf16)(x0[0] * f), (__bf16)(x0[1] * f), (__bf16)(x1[0] * f), (__bf16)(x1[1] * f),
              (__bf16)(x2[0] * f), (__bf16)(x2[1] * f), (__bf16)(x3[0] * f), (__bf16)(x3[1] * f)};
#else
  (void)codes;
  (void)scale;
  return v8bf{};
#endif
}

template <int kNV, int MT>
__global__ void __launch_bounds__(256) gemm_w4a16_kernel(W16Args a) {
  using namespace w16;
  // per wave: four fragment staging areas in the loop, then MT x 16 x 64 fp32 partial sums
  constexpr int kWaveBytes = 4 * kStgBytes > MT * 4096 ? 4 * kStgBytes : MT * 4096;
  __shared__ v4i lds[4][kWaveBytes / 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int m = (int)a.M;
  const int64_t K = a.K, wrow = K / 2, srow = kNV ? K / 16 : K / 32;
  const int sb_ss = kNV ? 32 : 16;  // scale bytes per row per super-step

  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t span = min((int64_t)64, a.N - n0);
  int roff[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) roff[f] = 16 * f < span ? 16 * f : 0;  // a fragment past N re-reads the first
  const buf_rsrc wr = make_rsrc(a.w + n0 * wrow, (uint32_t)(span * wrow));
  const buf_rsrc sr = make_rsrc(a.ws + n0 * srow, (uint32_t)(span * srow));
  const int q = lane >> 3, rot = ((lane & 7) + q) & 7;
  const uint32_t wvoff = (uint32_t)(q * wrow + 16 * rot);
  const uint32_t svoff = (uint32_t)(r16 * srow);
  uint8_t* const stg = reinterpret_cast<uint8_t*>(&lds[wave][0]);
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    rd[s] = (2 * (s >> 1) + (r16 >> 3)) * kStgStride + 128 * (r16 & 7) + 16 * ((4 * s + g - (r16 & 7)) & 7);
  // activation rows of the MT fragments; rows past m read row m - 1 (their outputs are not stored)
  const uint16_t* ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) ap[mt] = a.a + (int64_t)min(16 * mt + r16, m - 1) * K + 8 * (4 * g);

  v4f acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nss = (int)(K / 512);
  int ss_lo = 0, ss_hi = nss;
  if (a.kchunk > 0) {
    ss_lo = (int)blockIdx.y * a.kchunk;
    ss_hi = min(nss, ss_lo + a.kchunk);
  }
  const int len = ss_hi - ss_lo;
  const int ss_begin = ss_lo + wave * len / 4, ss_end = ss_lo + (wave + 1) * len / 4;
  for (int ss = ss_begin; ss < ss_end; ++ss) {
    // the super-step's 16 weight lines and scale bytes, all in flight before any wait
    v4i raw[4][4], sraw[4][2];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int ro = roff[f];
#pragma unroll
      for (int h = 0; h < (kNV ? 2 : 1); ++h)
        sraw[f][h] = buf_load16(sr, svoff, (uint32_t)(ro * srow + ss * sb_ss + 16 * h));
#pragma unroll
      for (int s = 0; s < 4; ++s)
        raw[f][s] = buf_load16_nt(wr, wvoff + 128 * (s >> 1), (uint32_t)((ro + 8 * (s & 1)) * wrow + ss * 256));
    }
    __builtin_amdgcn_sched_barrier(0);
    // into the matrix lane layout: lane (g, r16) gets row r16, block 4 s + g at step s
    v4i b[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      uint8_t* const area = stg + f * kStgBytes;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<v4i*>(area + s * kStgStride + 16 * lane) = raw[f][s];
#pragma unroll
      for (int s = 0; s < 4; ++s) b[f][s] = *reinterpret_cast<const v4i*>(area + rd[s]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i av[MT][4];  // activations of step s: k = 512 ss + 32 (4 s + g) + 8 j + [0, 8)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          av[mt][j] = *reinterpret_cast<const v4i*>(ap[mt] + (int64_t)ss * 512 + 128 * s + 8 * j);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        // scale of block 4 s + g of this lane's row (NVFP4: one per 16 codes, so
        // instructions j = 0, 1 take the first, j = 2, 3 the second)
        float sc[2];
        if (kNV) {
          const int byte = 2 * (4 * s + g);  // 0 .. 31 of the super-step's 32 scale bytes
          const uint32_t dw = (uint32_t)sraw[f][byte >> 4][(byte >> 2) & 3];
          sc[0] = ue4m3_to_f32((dw >> (8 * (byte & 3))) & 0xFFu);
          sc[1] = ue4m3_to_f32((dw >> (8 * ((byte & 3) + 1))) & 0xFFu);
        } else {
          const int byte = 4 * s + g;
          const uint32_t dw = (uint32_t)sraw[f][0][byte >> 2];
          sc[0] = sc[1] = ue8m0_to_f32((dw >> (8 * (byte & 3))) & 0xFFu);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v8bf wv = kNV ? decode8_nv((uint32_t)b[f][s][j], sc[j >> 1]) : decode8((uint32_t)b[f][s][j], sc[0]);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, av[mt][j]), wv,
                                                                 acc[mt][f], 0, 0, 0);
        }
      }
    }
  }

  float* const out = a.kchunk > 0 ? a.out + (int64_t)blockIdx.y * a.M * a.N : a.out;
  // the 4 waves' K shares summed in a fixed order (deterministic); acc[mt][f][v] is
  // token row 16 mt + 4 g + v, weight row 16 f + r16
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        reinterpret_cast<float*>(&lds[wave][0])[((mt * 16) + f * 4 + v) * 64 + lane] = acc[mt][f][v];
  __syncthreads();
  for (int mt = wave; mt < MT; mt += 4) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float* r = reinterpret_cast<const float*>(&lds[0][0]) + ((mt * 16) + f * 4 + v) * 64 + lane;
        constexpr int kW = kWaveBytes / 4;
        const float tot = ((r[0] + r[kW]) + r[2 * kW]) + r[3 * kW];
        const int lr = 16 * mt + 4 * g + v;
        if (lr < m && 16 * f < span) out[(int64_t)lr * a.N + n0 + 16 * f + r16] = tot;
      }
  }
}

int w4a16_ksplit(int64_t M, int64_t N, int64_t K) {
  // 64 weight rows per workgroup: for narrow N also split K in slices of 4 super-steps
  (void)M;
  const int64_t nss = K / 512;
  return N / 64 >= 256 || nss <= 4 ? 1 : (int)cdiv(nss, 4);
}

template <int kNV>
static void launch_w4a16_mt(const W16Args& a, int mt, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 1: gemm_w4a16_kernel<kNV, 1><<<grid, 256, 0, stream>>>(a); break;
    case 2: gemm_w4a16_kernel<kNV, 2><<<grid, 256, 0, stream>>>(a); break;
    case 3: gemm_w4a16_kernel<kNV, 3><<<grid, 256, 0, stream>>>(a); break;
    default: gemm_w4a16_kernel<kNV, 4><<<grid, 256, 0, stream>>>(a); break;
  }
}

int launch_w4a16_gemm(bool nvfp4, const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                      const uint8_t* ws, float* c, float* partials, hipStream_t stream) {
  const int S = w4a16_ksplit(M, N, K);
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int64_t mm = M - m0 < 64 ? M - m0 : 64;
    W16Args args{a + m0 * K, w, ws, S > 1 ? partials : c + m0 * N, mm, N, K, S > 1 ? 4 : 0};
    const dim3 grid((unsigned)cdiv(N, 64), (unsigned)S);
    if (nvfp4) launch_w4a16_mt<1>(args, (int)cdiv(mm, 16), grid, stream);
    else launch_w4a16_mt<0>(args, (int)cdiv(mm, 16), grid, stream);
    if (S > 1) launch_reduce_partials(partials, S, mm * N, c + m0 * N, stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

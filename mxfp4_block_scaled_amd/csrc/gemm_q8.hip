// The lookup-table route: Q8 activations x MXFP4 weights through int8 products.
//
// Hardware without FP4 matrix instructions runs FP4 weights through its int8 path:
// the weights are expanded to int8 by a 16-entry table and the activations quantised
// to Q8 (32 int8 values and one fp16 scale per block), lossless on the weight side
// and with no FP4 speed bonus (page "DGX Spark 原生 FP4 矩阵指令" sections 二 and 三;
// FP4 and the 4-bit lookup-table types are interchangeable through such a table, page
// "企业官网建设流程全解析" section 五). Here:
//   activations: per 32-block d = fp16(amax / 127), q = clamp(rne(x / d), -127, 127),
//                both quotients in fp32 (q = 0 where d = 0);
//   weights:     int8 = 2 x e2m1(code) in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12}, block
//                scale 2^(byte - 128), so int8 x scale is the MXFP4 value exactly;
//   C[m][n] = sum over blocks b of (sum_k q[m][k] w8[n][k]) x d[m][b] x 2^(e[n][b] - 128):
//                the integer sum of a block (at most 32 x 127 x 12) is exact in int32 and
//                in fp32, each block's scaling and the sum over blocks round in fp32.
// One 16x16x32 int8 matrix instruction covers exactly one 32-block, so the block's
// integer sum comes out whole and is scaled on the VALU.
//
// Weight streaming as in the other streaming kernels: whole 128-byte lines through a
// per-wave LDS area; a lane then reads the 4 bytes (8 codes) of its row, block b,
// elements 8 g .. 8 g + 7 - the instruction's lane group g - and expands them to int8
// with two byte permutes per 4 codes.
#include "gemm_common.hpp"

namespace mxf {

namespace q8 {
constexpr int kStgStride = 1152;
constexpr int kStgBytes = 4 * kStgStride;
}  // namespace q8

// ---------------------------------------------------------------------------------
// Q8 activation quantisation: one thread per 32-block (64 bytes of bf16 in, 32 int8 and
// one fp16 scale out)
__global__ void __launch_bounds__(256) q8_quantize_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                          int8_t* __restrict__ q, uint16_t* __restrict__ d) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = src[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = __uint_as_float(ws[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(ws[j] & 0xFFFF0000u);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const _Float16 dh = (_Float16)(amax / 127.0f);  // fp32 quotient, rounded to fp16 (nearest even)
  const float df = (float)dh;
  uint32_t out[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float t = df > 0.0f ? __builtin_rintf(v[4 * w + n] / df) : 0.0f;
      const int qi = (int)fminf(fmaxf(t, -127.0f), 127.0f);
      word |= ((uint32_t)qi & 0xFFu) << (8 * n);
    }
    out[w] = word;
  }
  uint4* dst = reinterpret_cast<uint4*>(q + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  d[b] = __builtin_bit_cast(uint16_t, dh);
}

int launch_q8_quantize(const uint16_t* x, int64_t rows, int64_t K, int8_t* q, uint16_t* d, hipStream_t stream) {
  const int64_t nblocks = rows * (K / 32);
  if (nblocks == 0) return 0;
  q8_quantize_kernel<<<(unsigned)cdiv(nblocks, 256), 256, 0, stream>>>(x, nblocks, q, d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------------
// 4 E2M1 codes (low nibbles of the 4 bytes of w) -> 4 int8 = 2 x e2m1: magnitudes and
// their negatives by byte permutes of 8-entry tables, chosen per byte by the sign bit
__device__ __forceinline__ uint32_t e2m1x4_to_i8(uint32_t w) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t mag = w & 0x07070707u;
  const uint32_t pos = __builtin_amdgcn_perm(0x0C080604u, 0x03020100u, mag);  // 0 1 2 3 | 4 6 8 12
  const uint32_t neg = __builtin_amdgcn_perm(0xF4F8FAFCu, 0xFDFEFF00u, mag);  // their negatives
  const uint32_t mask = ((w >> 3) & 0x01010101u) * 0xFFu;
  return (pos & ~mask) | (neg & mask);
#else
  return w;
#endif
}

// 8 codes (one dword, element 2 n in the low nibble of byte n) -> 8 int8 in element order
__device__ __forceinline__ long e2m1x8_to_i8(uint32_t c) {
  const uint32_t lo = e2m1x4_to_i8(c & 0x0F0F0F0Fu);         // elements 0, 2, 4, 6
  const uint32_t hi = e2m1x4_to_i8((c >> 4) & 0x0F0F0F0Fu);  // elements 1, 3, 5, 7
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t e03 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  const uint32_t e47 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
#else
  const uint32_t e03 = lo, e47 = hi;
#endif
  return (long)(((uint64_t)e47 << 32) | e03);
}

struct Q8Args {
  const int8_t* q;    // [M][K]
  const uint16_t* d;  // [M][K/32] fp16
  const uint8_t* w;   // [N][K/2]
  const uint8_t* ws;  // [N][K/32]
  float* out;         // [M][N] or [slices][M][N]
  int64_t M, N, K;
  int kchunk;
};

template <int MT>
__global__ void __launch_bounds__(256) gemm_q8_kernel(Q8Args a) {
  using namespace q8;
  constexpr int kWaveBytes = 4 * kStgBytes > MT * 4096 ? 4 * kStgBytes : MT * 4096;
  __shared__ v4i lds[4][kWaveBytes / 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int m = (int)a.M;
  const int64_t K = a.K, wrow = K / 2, srow = K / 32;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t span = min((int64_t)64, a.N - n0);
  int roff[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) roff[f] = 16 * f < span ? 16 * f : 0;
  const buf_rsrc wr = make_rsrc(a.w + n0 * wrow, (uint32_t)(span * wrow));
  const buf_rsrc sr = make_rsrc(a.ws + n0 * srow, (uint32_t)(span * srow));
  const int qq = lane >> 3, rot = ((lane & 7) + qq) & 7;
  const uint32_t wvoff = (uint32_t)(qq * wrow + 16 * rot);
  const uint32_t svoff = (uint32_t)(r16 * srow);
  uint8_t* const stg = reinterpret_cast<uint8_t*>(&lds[wave][0]);
  // where 16-byte chunk c of row r16's super-step segment landed in a staging area
  auto chunk_at = [&](int c) {
    return (2 * (c >> 3) + (r16 >> 3)) * kStgStride + 128 * (r16 & 7) + 16 * (((c & 7) - (r16 & 7)) & 7);
  };
  // activation rows (token fragment mt): lane (g, r16) supplies row 16 mt + r16, elements
  // 8 g .. 8 g + 7 of each block; the scaling uses the scales of rows 16 mt + 4 g + v
  const int8_t* ap[MT];
  const uint16_t* dp[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    ap[mt] = a.q + (int64_t)min(16 * mt + r16, m - 1) * K + 8 * g;
#pragma unroll
    for (int v = 0; v < 4; ++v) dp[mt][v] = a.d + (int64_t)min(16 * mt + 4 * g + v, m - 1) * (K / 32);
  }
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
    v4i raw[4][4], sraw[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int ro = roff[f];
      sraw[f] = buf_load16(sr, svoff, (uint32_t)(ro * srow + ss * 16));
#pragma unroll
      for (int s = 0; s < 4; ++s)
        raw[f][s] = buf_load16_nt(wr, wvoff + 128 * (s >> 1), (uint32_t)((ro + 8 * (s & 1)) * wrow + ss * 256));
    }
    // the activation scales of the super-step's 16 blocks for this lane's 4 token rows
    v4i draw[MT][4][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int h = 0; h < 2; ++h) draw[mt][v][h] = *reinterpret_cast<const v4i*>(dp[mt][v] + ss * 16 + 8 * h);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      uint8_t* const area = stg + f * kStgBytes;
#pragma unroll
      for (int s = 0; s < 4; ++s) *reinterpret_cast<v4i*>(area + s * kStgStride + 16 * lane) = raw[f][s];
    }
#pragma unroll 4
    for (int b = 0; b < 16; ++b) {
      long av[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[mt] = *reinterpret_cast<const long*>(ap[mt] + (int64_t)ss * 512 + 32 * b);
      float da[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t word = (uint32_t)draw[mt][v][b >> 3][(b >> 1) & 3];
          const uint16_t hb = (uint16_t)(word >> (16 * (b & 1)));
          da[mt][v] = (float)__builtin_bit_cast(_Float16, hb);
        }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint32_t codes = *reinterpret_cast<const uint32_t*>(stg + f * kStgBytes + chunk_at(b) + 4 * g);
        const long wv = e2m1x8_to_i8(codes);
        const uint32_t sbyte = ((uint32_t)sraw[f][b >> 2] >> (8 * (b & 3))) & 0xFFu;
        const float dw = __uint_as_float(sbyte > 1u ? (sbyte - 1u) << 23 : (0x00400000u >> (1u - sbyte)));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const v4i ib = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[mt], wv, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mt][f][v] = fmaf((float)ib[v], da[mt][v] * dw, acc[mt][f][v]);
        }
      }
    }
  }

  float* const out = a.kchunk > 0 ? a.out + (int64_t)blockIdx.y * a.M * a.N : a.out;
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

template <int MT>
static void launch_q8_t(const Q8Args& a, dim3 grid, hipStream_t stream) {
  gemm_q8_kernel<MT><<<grid, 256, 0, stream>>>(a);
}

int launch_q8_gemm(const int8_t* q, const uint16_t* d, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                   const uint8_t* ws, float* c, float* partials, hipStream_t stream) {
  const int S = w4a16_ksplit(M, N, K);  // the same K slicing as the bf16-activation kernel
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int64_t mm = M - m0 < 64 ? M - m0 : 64;
    Q8Args args{q + m0 * K, d + m0 * (K / 32), w, ws, S > 1 ? partials : c + m0 * N, mm, N, K, S > 1 ? 4 : 0};
    const dim3 grid((unsigned)cdiv(N, 64), (unsigned)S);
    switch ((int)cdiv(mm, 16)) {
      case 1: launch_q8_t<1>(args, grid, stream); break;
      case 2: launch_q8_t<2>(args, grid, stream); break;
      case 3: launch_q8_t<3>(args, grid, stream); break;
      default: launch_q8_t<4>(args, grid, stream); break;
    }
    if (S > 1) launch_reduce_partials(partials, S, mm * N, c + m0 * N, stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

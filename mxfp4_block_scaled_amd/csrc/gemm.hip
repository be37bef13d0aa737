// MXFP4 expert GEMMs on gfx950 scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// The weights stay E2M1 + UE8M0 all the way into the matrix instruction - no
// dequantisation to a 16-bit type (page "DGX Spark 原生 FP4 矩阵指令" sections 一
// and 二; the pages' point that removing data movement beats faster compute,
// "【DeepSeek V4】Triton FP4 优化实战" 第二步). Activations are E4M3 (FP8 x FP4)
// or E2M1 (FP4 x FP4); products are exact and accumulate in fp32.
//
// K ordering. The instruction contracts over 128 "hardware" k per step; which
// memory k feed them is ours to choose, as long as both operands and their
// scales agree. Within a super-step of S MFMA steps (S*128 memory k, S*4
// memory blocks of 32), hardware block hb of step s reads memory block S*hb+s.
// Then an FP4 lane of lane-group g reads S contiguous 16-byte chunks of its row
// across the super-step, and its S scale bytes are contiguous too: one
// 32-bit (S = 4) or 16-bit (S = 2) scale load per row, op_sel = s picks the
// byte. For an FP8 operand the lane's two 16-byte halves come from memory
// blocks S*(g/2)+s and S*(2+g/2)+s, half g&1 (see the layout in common.hpp).
//
// Two kernels:
//  * gemm_stream_kernel - few rows per expert (decode, small dense M): weights
//    go straight from HBM to registers in the instruction's lane layout
//    (64 contiguous bytes per lane per 512-k super-step), the K range is split
//    over the 4 waves and reduced through LDS. One workgroup = one expert x
//    64 weight rows (FC1: 32 gate + 32 matching up rows).
//  * gemm_tile_kernel - many rows per expert (prefill): 128 x 128 output tile,
//    256-k stages double-buffered in LDS (XOR-swizzled 16-byte chunks), each
//    of the 4 waves computes 64 x 64 with 4 x 4 MFMA tiles.
// FC1's epilogue fuses SwiGLU and the requantisation of h per 32 along I
// (page "Domestic GPUs are awesome! ... DeepSeek-V4": "SwiGLU + FP8 quant").
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
  int topk, E;
  int ntiles;  // tile kernel: weight-row tiles per expert (1-D grid: block = m_unit * ntiles + n_tile)
};

// ---------------------------------------------------------------------------------
// Which expert does work unit u belong to? units(e) = (count_e > 0) when BM == 0,
// else ceil(count_e / BM). Called by a whole wave; results are wave-uniform.
template <int BM>
__device__ __forceinline__ int units_of(int c) {
  if constexpr (BM == 0) return c > 0 ? 1 : 0;
  else return (c + BM - 1) / BM;
}

template <int BM>
__device__ __forceinline__ void find_unit(const int32_t* __restrict__ off, int E, int u, int& e_out, int& loc_out) {
  const int lane = threadIdx.x & 63;
  const int C = (E + 63) >> 6;
  const int first = lane * C;
  int units = 0;
  for (int i = 0; i < C; ++i) {
    const int e = first + i;
    if (e < E) {
      const int c = off[e + 1] - off[e];
      units += units_of<BM>(c);
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
        const int n = units_of<BM>(c);
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

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// FC1 epilogue for one 16-row m-fragment held as tot[f][v], f = gate0, gate1, up0, up1,
// lane (g = l/16, r16 = l%16): row 4g+v, column i_base + 16*(f&1) + r16.
// The 32 columns [i_base, i_base+32) form exactly one quantisation block.
template <bool kActFP4>
__device__ __forceinline__ void epilogue_fc1(const float (&tot)[4][4], int local_row0, int m_valid, int64_t row_base,
                                             int64_t i_base, int64_t I, uint8_t* __restrict__ h,
                                             uint8_t* __restrict__ h_scale) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float hv[2];
    hv[0] = silu_mul(tot[0][v], tot[2][v]);
    hv[1] = silu_mul(tot[1][v], tot[3][v]);
    uint32_t amax = max(__float_as_uint(hv[0]) & 0x7FFFFFFFu, __float_as_uint(hv[1]) & 0x7FFFFFFFu);
    amax = __float_as_uint(wave_max16(__uint_as_float(amax)));
    const uint32_t byte = scale_byte_from_amax_bits(amax, kActFP4 ? kEmaxE2M1 : kEmaxE4M3);
    const float inv = inv_scale_from_byte(byte);
    uint32_t code[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) code[c] = kActFP4 ? e2m1_code(hv[c], inv) : e4m3_code(hv[c], inv);
    uint32_t pair[2];
    if (kActFP4) {
#pragma unroll
      for (int c = 0; c < 2; ++c) pair[c] = code[c] | (__shfl_xor(code[c], 1) << 4);
    }
    const int lr = local_row0 + 4 * g + v;
    if (lr < m_valid) {
      const int64_t R = row_base + lr;
      if (kActFP4) {
        if ((r16 & 1) == 0) {
#pragma unroll
          for (int c = 0; c < 2; ++c) h[R * (I / 2) + (i_base + 16 * c + r16) / 2] = (uint8_t)pair[c];
        }
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) h[R * I + i_base + 16 * c + r16] = (uint8_t)code[c];
      }
      if (r16 == 0) h_scale[R * (I / 32) + i_base / 32] = (uint8_t)byte;
    }
  }
}

template <bool kYBF16>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float x) {
  if (kYBF16)
    static_cast<uint16_t*>(out)[idx] = (uint16_t)bf16_round(x);
  else
    static_cast<float*>(out)[idx] = x;
}

// ---------------------------------------------------------------------------------
// weight-streaming kernel (rows per expert <= 16 * MT)
//
// K order inside a 512-k super-step: step s, hardware block hb <-> memory block
// 4 s + hb. Then the 4 lane groups of a row read 64 contiguous bytes per load
// instruction (16 bytes each, FP4), and an FP8 lane's two 16-byte halves sit at
// 128 s + 16 g and 128 s + 64 + 16 g. The scale of (row, block 4 s + g) is byte
// 4 s + g of the row's 16 scale bytes, so a lane gathers bytes g, 4+g, 8+g and
// 12+g of them into one register (op_sel = s picks byte s).
__device__ __forceinline__ int gather_scales(v4i d, int g) {
  const int sh = 8 * g;
  return (int)((((uint32_t)d[0] >> sh) & 0xFFu) | ((((uint32_t)d[1] >> sh) & 0xFFu) << 8) |
               ((((uint32_t)d[2] >> sh) & 0xFFu) << 16) | ((((uint32_t)d[3] >> sh) & 0xFFu) << 24));
}

template <bool kActFP4, int kMode, bool kYBF16, int MT>
__global__ void __launch_bounds__(256) gemm_stream_kernel(GemmArgs a) {
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  __shared__ float red[4][MT * 16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;

  int e = 0;
  int64_t row0 = 0;
  int m = 0;
  if (kMode == kModeDense) {
    m = (int)a.M;
  } else {
    int loc;
    find_unit<0>(a.offsets, a.E, blockIdx.y, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e];
    m = a.offsets[e + 1] - (int)row0;
  }
  const int64_t K = a.K;
  const int64_t wrow_bytes = K / 2, srow_bytes = K / 32;
  const int64_t arow_bytes = kActFP4 ? K / 2 : K;

  // the 4 weight fragments of this workgroup
  const uint8_t* wp[4];
  const uint8_t* sp[4];
  bool fvalid[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    int64_t n;
    if (kMode == kModeFC1) {
      const int64_t i0 = (int64_t)blockIdx.x * 32 + 16 * (f & 1);
      n = (f < 2 ? 0 : a.I) + i0;
      fvalid[f] = true;
    } else {
      n = (int64_t)blockIdx.x * 64 + 16 * f;
      fvalid[f] = n < a.N;
    }
    const int64_t nr = n + r16;
    wp[f] = a.w + ((int64_t)e * a.N + nr) * wrow_bytes + 16 * g;
    sp[f] = a.w_scale + ((int64_t)e * a.N + nr) * srow_bytes;
  }
  // activation rows of the MT fragments
  const uint8_t* ap[MT];
  const uint8_t* asp[MT];
  bool avalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int lr = 16 * mt + r16;
    avalid[mt] = lr < m;
    int64_t src = 0;
    if (avalid[mt]) {
      if (kMode == kModeFC1) src = a.sorted_pair[row0 + lr] / a.topk;
      else src = row0 + lr;
    }
    ap[mt] = a.act + src * arow_bytes + 16 * g;
    asp[mt] = a.act_scale + src * srow_bytes;
  }

  v4f acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[mt][f] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nss = (int)(K / 512);
  const int ss_begin = wave * nss / 4, ss_end = (wave + 1) * nss / 4;
  for (int ss = ss_begin; ss < ss_end; ++ss) {
    v4i bq[4][4];
    int bs[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (fvalid[f]) {
        const uint8_t* src = wp[f] + (int64_t)ss * 256;
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[f][s] = *reinterpret_cast<const v4i*>(src + 64 * s);
        bs[f] = gather_scales(*reinterpret_cast<const v4i*>(sp[f] + (int64_t)ss * 16), g);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[f][s] = v4i{0, 0, 0, 0};
        bs[f] = 0;
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      v8i aq[4];
      int as = 0;
      if (avalid[mt]) {
        if (kActFP4) {
          const uint8_t* src = ap[mt] + (int64_t)ss * 256;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            v4i x = *reinterpret_cast<const v4i*>(src + 64 * s);
            aq[s] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
          }
        } else {
          const uint8_t* base = ap[mt] + (int64_t)ss * 512;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            v4i lo = *reinterpret_cast<const v4i*>(base + 128 * s);
            v4i hi = *reinterpret_cast<const v4i*>(base + 128 * s + 64);
            aq[s] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
        as = gather_scales(*reinterpret_cast<const v4i*>(asp[mt] + (int64_t)ss * 16), g);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) aq[s] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        v8i b0 = v8i{bq[f][0][0], bq[f][0][1], bq[f][0][2], bq[f][0][3], 0, 0, 0, 0};
        v8i b1 = v8i{bq[f][1][0], bq[f][1][1], bq[f][1][2], bq[f][1][3], 0, 0, 0, 0};
        v8i b2 = v8i{bq[f][2][0], bq[f][2][1], bq[f][2][2], bq[f][2][3], 0, 0, 0, 0};
        v8i b3 = v8i{bq[f][3][0], bq[f][3][1], bq[f][3][2], bq[f][3][3], 0, 0, 0, 0};
        acc[mt][f] = mfma16x16x128<kFA, kFmtFP4, 0>(aq[0], b0, acc[mt][f], as, bs[f]);
        acc[mt][f] = mfma16x16x128<kFA, kFmtFP4, 1>(aq[1], b1, acc[mt][f], as, bs[f]);
        acc[mt][f] = mfma16x16x128<kFA, kFmtFP4, 2>(aq[2], b2, acc[mt][f], as, bs[f]);
        acc[mt][f] = mfma16x16x128<kFA, kFmtFP4, 3>(aq[3], b3, acc[mt][f], as, bs[f]);
      }
    }
  }

  // reduce the 4 K-slices in a fixed order (deterministic)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][mt * 16 + f * 4 + v][lane] = acc[mt][f][v];
  __syncthreads();
  for (int mt = wave; mt < MT; mt += 4) {
    float tot[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int idx = mt * 16 + f * 4 + v;
        tot[f][v] = ((red[0][idx][lane] + red[1][idx][lane]) + red[2][idx][lane]) + red[3][idx][lane];
      }
    if (kMode == kModeFC1) {
      epilogue_fc1<kActFP4>(tot, 16 * mt, m, row0, (int64_t)blockIdx.x * 32, a.I, a.h, a.h_scale);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int lr = 16 * mt + 4 * g + v;
        if (lr < m) {
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const int64_t n = (int64_t)blockIdx.x * 64 + 16 * f + r16;
            if (fvalid[f]) store_out<kYBF16>(a.out, (row0 + lr) * a.N + n, tot[f][v]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// LDS-tiled kernel: 128 rows x 128 weight rows, 256-k stages, double-buffered.
constexpr int kBM = 128, kBN = 128, kStageK = 256;

__device__ __forceinline__ int swz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <bool kActFP4>
struct alignas(16) TileSmem {
  static constexpr int kArow = kActFP4 ? kStageK / 2 : kStageK;  // bytes per A row per stage
  uint8_t A[2][kBM * kArow];
  uint8_t B[2][kBN * (kStageK / 2)];
  uint8_t As[2][kBM * 8];
  uint8_t Bs[2][kBN * 8];
};

template <bool kActFP4, int kMode, bool kYBF16>
__global__ void __launch_bounds__(256) gemm_tile_kernel(GemmArgs a) {
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  constexpr int kArow = TileSmem<kActFP4>::kArow;
  constexpr int kAChunks = kArow / 16;                 // 16-byte chunks per A row per stage (8 or 16)
  constexpr int kAPerThread = kBM * kAChunks / 256;    // 4 or 8
  constexpr int kBPerThread = kBN * 8 / 256;           // 4
  __shared__ TileSmem<kActFP4> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  const int n_tile = (int)(blockIdx.x % (unsigned)a.ntiles);
  const int m_unit = (int)(blockIdx.x / (unsigned)a.ntiles);

  int e = 0;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
    row0 = (int64_t)m_unit * kBM;
    if (row0 >= a.M) return;
    m = (int)(a.M - row0 < kBM ? a.M - row0 : kBM);
  } else {
    int loc;
    find_unit<kBM>(a.offsets, a.E, m_unit, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e] + (int64_t)loc * kBM;
    m = min(kBM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t wrow_bytes = K / 2, srow_bytes = K / 32;
  const int64_t arow_bytes = kActFP4 ? K / 2 : K;

  // global sources of this thread's A chunks (gathered rows for FC1)
  const uint8_t* a_src[kAPerThread];
  bool a_ok[kAPerThread];
  const int a_c = tid % kAChunks;
#pragma unroll
  for (int j = 0; j < kAPerThread; ++j) {
    const int r = tid / kAChunks + j * (256 / kAChunks);
    a_ok[j] = r < m;
    int64_t src = 0;
    if (a_ok[j]) src = (kMode == kModeFC1) ? a.sorted_pair[row0 + r] / a.topk : row0 + r;
    a_src[j] = a.act + src * arow_bytes + 16 * a_c;
  }
  // B chunks
  const uint8_t* b_src[kBPerThread];
  const int b_c = tid & 7;
#pragma unroll
  for (int j = 0; j < kBPerThread; ++j) {
    const int r = (tid >> 3) + j * 32;
    int64_t n;
    if (kMode == kModeFC1) n = (r < 64 ? 0 : a.I - 64) + (int64_t)n_tile * 64 + r;
    else n = (int64_t)n_tile * kBN + r;
    b_src[j] = a.w + ((int64_t)e * a.N + n) * wrow_bytes + 16 * b_c;
  }
  // scales: threads 0..127 load A row tid, 128..255 load B row tid-128 (8 bytes per stage)
  const uint8_t* s_src;
  bool s_ok = true;
  {
    if (tid < 128) {
      s_ok = tid < m;
      int64_t src = 0;
      if (s_ok) src = (kMode == kModeFC1) ? a.sorted_pair[row0 + tid] / a.topk : row0 + tid;
      s_src = a.act_scale + src * srow_bytes;
    } else {
      const int r = tid - 128;
      int64_t n;
      if (kMode == kModeFC1) n = (r < 64 ? 0 : a.I - 64) + (int64_t)n_tile * 64 + r;
      else n = (int64_t)n_tile * kBN + r;
      s_src = a.w_scale + ((int64_t)e * a.N + n) * srow_bytes;
    }
  }

  v4i ra[kAPerThread], rb[kBPerThread];
  uint2 rs;
  auto gload = [&](int st) {
    const int64_t aoff = (int64_t)st * kArow, boff = (int64_t)st * (kStageK / 2);
#pragma unroll
    for (int j = 0; j < kAPerThread; ++j)
      ra[j] = a_ok[j] ? *reinterpret_cast<const v4i*>(a_src[j] + aoff) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kBPerThread; ++j) rb[j] = *reinterpret_cast<const v4i*>(b_src[j] + boff);
    rs = s_ok ? *reinterpret_cast<const uint2*>(s_src + (int64_t)st * 8) : make_uint2(0, 0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kAPerThread; ++j) {
      const int r = tid / kAChunks + j * (256 / kAChunks);
      const int pc = kActFP4 ? (a_c ^ swz8(r)) : (a_c ^ (r & 15));
      *reinterpret_cast<v4i*>(&sm.A[buf][r * kArow + 16 * pc]) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < kBPerThread; ++j) {
      const int r = (tid >> 3) + j * 32;
      *reinterpret_cast<v4i*>(&sm.B[buf][r * 128 + 16 * (b_c ^ swz8(r))]) = rb[j];
    }
    if (tid < 128) *reinterpret_cast<uint2*>(&sm.As[buf][tid * 8]) = rs;
    else *reinterpret_cast<uint2*>(&sm.Bs[buf][(tid - 128) * 8]) = rs;
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // LDS row of each fragment this lane reads
  int arow[4], brow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    arow[f] = 64 * wm + 16 * f + r16;
    if (kMode == kModeFC1) brow[f] = (f < 2 ? 0 : 64) + 32 * wn + 16 * (f & 1) + r16;
    else brow[f] = 64 * wn + 16 * f + r16;
  }

  const int nst = (int)(K / kStageK);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) gload(st + 1);
    int sa[4], sb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sa[f] = *reinterpret_cast<const uint16_t*>(&sm.As[buf][arow[f] * 8 + 2 * g]);
      sb[f] = *reinterpret_cast<const uint16_t*>(&sm.Bs[buf][brow[f] * 8 + 2 * g]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v8i af[4], bf[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int r = arow[f];
        if (kActFP4) {
          const int c = 2 * g + s;
          v4i x = *reinterpret_cast<const v4i*>(&sm.A[buf][r * kArow + 16 * (c ^ swz8(r))]);
          af[f] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
        } else {
          const int c1 = 2 * (2 * (g >> 1) + s) + (g & 1);
          const int c2 = 2 * (4 + 2 * (g >> 1) + s) + (g & 1);
          v4i lo = *reinterpret_cast<const v4i*>(&sm.A[buf][r * kArow + 16 * (c1 ^ (r & 15))]);
          v4i hi = *reinterpret_cast<const v4i*>(&sm.A[buf][r * kArow + 16 * (c2 ^ (r & 15))]);
          af[f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        const int rb2 = brow[f];
        const int cb = 2 * g + s;
        v4i y = *reinterpret_cast<const v4i*>(&sm.B[buf][rb2 * 128 + 16 * (cb ^ swz8(rb2))]);
        bf[f] = v8i{y[0], y[1], y[2], y[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int fm = 0; fm < 4; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          if (s == 0)
            acc[fm][fn] = mfma16x16x128<kFA, kFmtFP4, 0>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else
            acc[fm][fn] = mfma16x16x128<kFA, kFmtFP4, 1>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
        }
    }
    if (st + 1 < nst) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int fm = 0; fm < 4; ++fm) {
    float tot[4][4];
#pragma unroll
    for (int fn = 0; fn < 4; ++fn)
#pragma unroll
      for (int v = 0; v < 4; ++v) tot[fn][v] = acc[fm][fn][v];
    const int lr0 = 64 * wm + 16 * fm;
    if (kMode == kModeFC1) {
      epilogue_fc1<kActFP4>(tot, lr0, m, row0, (int64_t)n_tile * 64 + 32 * wn, a.I, a.h, a.h_scale);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int lr = lr0 + 4 * g + v;
        if (lr < m) {
#pragma unroll
          for (int fn = 0; fn < 4; ++fn) {
            const int64_t n = (int64_t)n_tile * kBN + 64 * wn + 16 * fn + r16;
            store_out<kYBF16>(a.out, (row0 + lr) * a.N + n, tot[fn][v]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// LDS-tiled kernel, 32x32x64 scaled MFMA: 128 rows x 256 weight rows per workgroup
// (4 waves of 64 x 128), KS-k stages double-buffered in LDS; the global loads of a
// stage are issued PD stages ahead into registers. LDS rows are padded by 16 B so
// the fragment reads of a wave hit distinct 16-byte bank groups.
//
// 32x32x64 operand layout: lane l holds row l%32; FP4 lanes hold hardware block
// g = l/32; FP8 lanes hold k in [16g, 16g+16) and [32+16g, 32+16g+16). Result:
// lane l holds C[8(v/4) + 4g + v%4][l%32], v = 0..15. A stage is S = KS/64 MFMA
// steps; hardware block hb of step s reads memory block S*hb + s, so a lane's S
// scale bytes are adjacent (at byte S*g; op_sel = s picks one).
#ifndef MXF_T2_KS
#define MXF_T2_KS 256
#endif
#ifndef MXF_T2_PD
#define MXF_T2_PD 1
#endif
#ifndef MXF_T2_XCD
#define MXF_T2_XCD 1
#endif
#ifndef MXF_TILE_V1
#define MXF_TILE_V1 0
#endif
#ifndef MXF_TILE_V3
#define MXF_TILE_V3 1
#endif
namespace t2 {
constexpr int BM = 128, BN = 256;
constexpr int KS = MXF_T2_KS;   // k per stage (128 or 256)
constexpr int PD = MXF_T2_PD;   // prefetch distance in stages (1 or 2)
constexpr int S = KS / 64;      // MFMA steps per stage
constexpr int kRowB = KS / 2 + 16;  // padded LDS bytes of an FP4 row
static_assert(KS == 128 || KS == 256, "stage k");
static_assert(PD == 1 || PD == 2, "prefetch distance");
}  // namespace t2

template <bool kActFP4>
struct alignas(16) Tile2Stage {
  static constexpr int kArow = (kActFP4 ? t2::KS / 2 : t2::KS) + 16;  // padded LDS bytes of an A row
  uint8_t A[2][t2::BM * kArow];
  uint8_t B[2][t2::BN * t2::kRowB];
  uint8_t As[2][t2::BM * (t2::KS / 32)];
  uint8_t Bs[2][t2::BN * (t2::KS / 32)];
};

template <bool kActFP4>
union alignas(16) Tile2Smem {
  Tile2Stage<kActFP4> st;
  uint16_t out[t2::BM][t2::BN + 8];      // bf16 epilogue staging (rows padded by 16 B)
  float hf[t2::BM][t2::BN / 2 + 4];      // FC1: fp32 h = silu(gate) * up (rows padded by 16 B)
  float of[t2::BM / 2][t2::BN + 4];      // fp32 output staging, one half of the rows at a time
};

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

template <bool kActFP4, int kMode, bool kYBF16>
__global__ void __launch_bounds__(256) gemm_tile2_kernel(GemmArgs a) {
  using namespace t2;
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  constexpr int kArow = Tile2Stage<kActFP4>::kArow;
  constexpr int kAC = (kActFP4 ? KS / 2 : KS) / 16;  // 16-byte chunks of an A row per stage
  constexpr int kAPT = BM * kAC / 256;               // A chunks per thread
  constexpr int kBC = KS / 32;                       // 16-byte chunks of a B row per stage
  constexpr int kBPT = BN * kBC / 256;               // B chunks per thread
  constexpr int kSB = KS / 32;                       // scale bytes per row per stage (4 or 8)
  __shared__ Tile2Smem<kActFP4> sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware order: block b runs on XCD b % 8. XCD x owns n-tiles [x*nt/8, (x+1)*nt/8);
  // its j-th block is m-unit j / nn, n-tile n_lo + j % nn, so consecutive blocks on an
  // XCD share A rows and the same n-tile recurs nn blocks later with the next m-unit.
  const int ntiles = a.ntiles;
#if MXF_T2_XCD
  const int x = (int)(blockIdx.x & 7u), j = (int)(blockIdx.x >> 3);
  const int n_lo = x * ntiles / 8, n_hi = (x + 1) * ntiles / 8, nn = n_hi - n_lo;
  if (nn == 0) return;
  const int m_unit = j / nn;
  const int n_tile = n_lo + j % nn;
#else
  const int m_unit = (int)(blockIdx.x / (unsigned)ntiles);
  const int n_tile = (int)(blockIdx.x % (unsigned)ntiles);
#endif

  int e = 0;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
    row0 = (int64_t)m_unit * BM;
    if (row0 >= a.M) return;
    m = (int)(a.M - row0 < BM ? a.M - row0 : BM);
  } else {
    int loc;
    find_unit<BM>(a.offsets, a.E, m_unit, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e] + (int64_t)loc * BM;
    m = min(BM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t wrow = K / 2, srow = K / 32;
  const int64_t arow = kActFP4 ? K / 2 : K;

  auto a_src_row = [&](int r) -> int64_t {
    return (kMode == kModeFC1) ? (int64_t)(a.sorted_pair[row0 + r] / a.topk) : row0 + r;
  };
  auto b_row = [&](int r) -> int64_t {
    if (kMode == kModeFC1) return (r < BN / 2 ? 0 : a.I - BN / 2) + (int64_t)n_tile * (BN / 2) + r;
    return (int64_t)n_tile * BN + r;
  };

  const uint8_t* a_src[kAPT];
  bool a_ok[kAPT];
  const int a_c = tid % kAC;
#pragma unroll
  for (int q = 0; q < kAPT; ++q) {
    const int r = tid / kAC + q * (256 / kAC);
    a_ok[q] = r < m;
    a_src[q] = a.act + (a_ok[q] ? a_src_row(r) : 0) * arow + 16 * a_c;
  }
  const uint8_t* b_src[kBPT];
  const int b_c = tid % kBC;
#pragma unroll
  for (int q = 0; q < kBPT; ++q) {
    const int r = tid / kBC + q * (256 / kBC);
    b_src[q] = a.w + ((int64_t)e * a.N + b_row(r)) * wrow + 16 * b_c;
  }
  const bool as_ok = tid < BM && tid < m;
  const uint8_t* as_src = a.act_scale + (as_ok ? a_src_row(tid) : 0) * srow;
  const uint8_t* bs_src = a.w_scale + ((int64_t)e * a.N + b_row(tid)) * srow;

  typedef typename std::conditional<kSB == 4, uint32_t, uint2>::type ScaleT;
  struct Regs {
    v4i ra[kAPT];
    v4i rb[kBPT];
    ScaleT sa, sb;
  };
  auto gload = [&](Regs& R, int st) {
    const int64_t ao = (int64_t)st * (kActFP4 ? KS / 2 : KS), bo = (int64_t)st * (KS / 2);
#pragma unroll
    for (int q = 0; q < kAPT; ++q)
      R.ra[q] = a_ok[q] ? *reinterpret_cast<const v4i*>(a_src[q] + ao) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < kBPT; ++q) R.rb[q] = *reinterpret_cast<const v4i*>(b_src[q] + bo);
    R.sa = as_ok ? *reinterpret_cast<const ScaleT*>(as_src + (int64_t)st * kSB) : ScaleT{};
    R.sb = *reinterpret_cast<const ScaleT*>(bs_src + (int64_t)st * kSB);
  };
  auto sstore = [&](const Regs& R, int buf) {
#pragma unroll
    for (int q = 0; q < kAPT; ++q) {
      const int r = tid / kAC + q * (256 / kAC);
      *reinterpret_cast<v4i*>(&sm.st.A[buf][r * kArow + 16 * a_c]) = R.ra[q];
    }
#pragma unroll
    for (int q = 0; q < kBPT; ++q) {
      const int r = tid / kBC + q * (256 / kBC);
      *reinterpret_cast<v4i*>(&sm.st.B[buf][r * kRowB + 16 * b_c]) = R.rb[q];
    }
    if (tid < BM) *reinterpret_cast<ScaleT*>(&sm.st.As[buf][tid * kSB]) = R.sa;
    *reinterpret_cast<ScaleT*>(&sm.st.Bs[buf][tid * kSB]) = R.sb;
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = v16f{};

  int arow_l[2], brow_l[4];
#pragma unroll
  for (int f = 0; f < 2; ++f) arow_l[f] = 64 * wm + 32 * f + r32;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if (kMode == kModeFC1) brow_l[f] = (f < 2 ? 0 : BN / 2) + 64 * wn + 32 * (f & 1) + r32;
    else brow_l[f] = 128 * wn + 32 * f + r32;
  }

  auto lds_scale = [&](const uint8_t* base) -> int {
    if (kSB == 4) return *reinterpret_cast<const uint16_t*>(base + 2 * g);
    return *reinterpret_cast<const int*>(base + 4 * g);
  };

  auto compute = [&](int buf) {
    int sa[2], sb[4];
#pragma unroll
    for (int f = 0; f < 2; ++f) sa[f] = lds_scale(&sm.st.As[buf][arow_l[f] * kSB]);
#pragma unroll
    for (int f = 0; f < 4; ++f) sb[f] = lds_scale(&sm.st.Bs[buf][brow_l[f] * kSB]);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      v8i af[2], bf[4];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const uint8_t* rowp = &sm.st.A[buf][arow_l[f] * kArow];
        if (kActFP4) {
          const v4i x4 = *reinterpret_cast<const v4i*>(rowp + 16 * (S * g + s));
          af[f] = v8i{x4[0], x4[1], x4[2], x4[3], 0, 0, 0, 0};
        } else {
          const v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (2 * s + g));
          const v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * (2 * (S + s) + g));
          af[f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const v4i y4 = *reinterpret_cast<const v4i*>(&sm.st.B[buf][brow_l[f] * kRowB + 16 * (S * g + s)]);
        bf[f] = v8i{y4[0], y4[1], y4[2], y4[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          if (s == 0) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 0>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 1) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 1>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 2) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 2>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 3>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
        }
    }
  };

  const int nst = (int)(K / KS);
  if (PD == 1) {
    // stage st computes from LDS buffer st&1 while the loads of stage st+1 are in flight
    Regs R;
    gload(R, 0);
    sstore(R, 0);
    lds_barrier();
    for (int st = 0; st < nst; ++st) {
      if (st + 1 < nst) gload(R, st + 1);
      compute(st & 1);
      if (st + 1 < nst) sstore(R, (st + 1) & 1);
      lds_barrier();
    }
  } else {
    // stage st computes from LDS buffer st&1 while registers hold stage st+1 (loaded an
    // iteration ago) and the loads of stage st+2 are in flight
    Regs R0, R1;
    gload(R0, 0);
    sstore(R0, 0);
    if (nst > 1) gload(R1, 1);
    lds_barrier();
    for (int st = 0; st < nst; st += 2) {
      if (st + 2 < nst) gload(R0, st + 2);
      compute(0);
      if (st + 1 < nst) sstore(R1, 1);
      lds_barrier();
      if (st + 1 >= nst) break;
      if (st + 3 < nst) gload(R1, st + 3);
      compute(1);
      if (st + 2 < nst) sstore(R0, 0);
      lds_barrier();
    }
  }

  // epilogues (the stage buffers are dead after the last barrier; the union reuses them)
  if (kMode == kModeFC1) {
    // h = silu(gate) * up in registers, fp32 h staged in LDS, then one thread per
    // (row, 32-column block) quantises and writes 16 / 32 contiguous bytes + 1 scale
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = 64 * wm + 32 * fm + 8 * (v >> 2) + 4 * g + (v & 3);
          sm.hf[rr][64 * wn + 32 * f + r32] = silu_mul(acc[fm][f][v], acc[fm][f + 2][v]);
        }
    __syncthreads();
    const int64_t i0 = (int64_t)n_tile * (BN / 2);
    const int64_t hrow = kActFP4 ? a.I / 2 : a.I;
#pragma unroll
    for (int q = 0; q < (BM * (BN / 2) / 32) / 256; ++q) {
      const int item = tid + 256 * q;
      const int rr = item >> 2, blk = item & 3;
      if (rr < m) {
        const int64_t R = row0 + rr;
        quantize_store32<kActFP4>(&sm.hf[rr][32 * blk], a.h + R * hrow + (i0 + 32 * blk) / (kActFP4 ? 2 : 1),
                                  a.h_scale + R * (a.I / 32) + i0 / 32 + blk);
      }
    }
  } else if (kYBF16) {
    // stage the 128 x 256 bf16 tile in LDS, then write whole 16-byte row segments
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = 64 * wm + 32 * fm + 8 * (v >> 2) + 4 * g + (v & 3);
          sm.out[rr][128 * wn + 32 * fn + r32] = (uint16_t)bf16_round(acc[fm][fn][v]);
        }
    __syncthreads();
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int q = 0; q < (BM * BN / 8) / 256; ++q) {
      const int idx = tid + 256 * q;
      const int rr = idx >> 5, cc = (idx & 31) * 8;
      if (rr < m) {
        const uint4 v = *reinterpret_cast<const uint4*>(&sm.out[rr][cc]);
        *reinterpret_cast<uint4*>(out + (row0 + rr) * a.N + (int64_t)n_tile * BN + cc) = v;
      }
    }
  } else {
    // fp32: stage one 64-row half at a time (the waves with wm == half), 16-byte stores
    float* out = static_cast<float*>(a.out);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int fn = 0; fn < 4; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rr = 32 * fm + 8 * (v >> 2) + 4 * g + (v & 3);
              sm.of[rr][128 * wn + 32 * fn + r32] = acc[fm][fn][v];
            }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < (BM / 2 * BN / 4) / 256; ++q) {
        const int idx = tid + 256 * q;
        const int rr = idx >> 6, cc = (idx & 63) * 4;
        const int lr = 64 * half + rr;
        if (lr < m)
          *reinterpret_cast<float4*>(out + (row0 + lr) * a.N + (int64_t)n_tile * BN + cc) =
              *reinterpret_cast<const float4*>(&sm.of[rr][cc]);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
// LDS-ring kernel, 32x32x64 scaled MFMA: 128 rows x 256 weight rows per workgroup
// (4 waves of 64 x 128). Operand tiles go HBM -> LDS with global_load_lds_dwordx4
// (no staging registers) into a ring of NS stage slots; the loads of stage st+NS-1
// are issued while stage st is computed, so NS-1 stages are in flight. Each slot is
// its own __shared__ object so the compiler can tell the slot being read from the
// slots being filled; lds_barrier() keeps the loads in flight across the barrier
// and an explicit vmcnt wait (counted in load instructions per wave) marks a
// stage as landed. 16-byte chunks are XOR-swizzled within a row: a lane of a DMA
// instruction writes LDS chunk p (fixed by its lane id) and fetches the global
// chunk that belongs there.
namespace t3 {
constexpr int BM = 128, BN = 256;
}  // namespace t3

template <bool kActFP4>
struct T3Cfg {
  static constexpr int KS = 256;                    // k per stage
  static constexpr int NS = kActFP4 ? 3 : 2;        // ring slots (a 3rd FP8 slot would not fit in LDS)
  static constexpr int S = KS / 64;                 // MFMA steps per stage
  static constexpr int RA = kActFP4 ? KS / 2 : KS;  // A bytes per row per stage
  static constexpr int RB = KS / 2;                 // B bytes per row per stage
  static constexpr int CA = RA / 16, CB = RB / 16;  // 16-byte chunks per row
  static constexpr int SB = KS / 32;                // scale bytes per row per stage
  static constexpr int IA = t3::BM * CA / 64 / 4;   // A DMA instructions per wave
  static constexpr int IB = t3::BN * CB / 64 / 4;   // B DMA instructions per wave
  static constexpr int ISA = t3::BM * SB / 256 / 4; // A-scale DMA instructions (4 B per lane) per wave
  static constexpr int ISB = t3::BN * SB / 256 / 4; // B-scale DMA instructions per wave
  static constexpr int D = IA + IB + ISA + ISB;      // DMA instructions per wave per stage
};

template <bool kActFP4>
struct alignas(16) T3Slot {
  uint8_t A[t3::BM * T3Cfg<kActFP4>::RA];
  uint8_t B[t3::BN * T3Cfg<kActFP4>::RB];
  uint8_t As[t3::BM * T3Cfg<kActFP4>::SB];
  uint8_t Bs[t3::BN * T3Cfg<kActFP4>::SB];
};

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

// NST > 0: the stage count K / 256 is a compile-time constant and the ring loop is
// fully unrolled (a runtime loop makes the compiler drain all loads once per ring
// turn); NST == 0: any K (multiple of 256) with a runtime loop.
template <bool kActFP4, int kMode, bool kYBF16, int NST>
__global__ void __launch_bounds__(256) gemm_tile3_kernel(GemmArgs a) {
  using namespace t3;
  using C = T3Cfg<kActFP4>;
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  struct alignas(16) NoSlot {
    uint8_t pad[16];
  };
  __shared__ T3Slot<kActFP4> slot0, slot1;
  __shared__ typename std::conditional<kActFP4, T3Slot<kActFP4>, NoSlot>::type slot2;  // 3rd slot: FP4 only

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 5, r32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware order (block b runs on XCD b % 8): XCD x owns n-tiles [x*nt/8, (x+1)*nt/8)
  const int ntiles = a.ntiles;
  const int x = (int)(blockIdx.x & 7u), jb = (int)(blockIdx.x >> 3);
  const int n_lo = x * ntiles / 8, n_hi = (x + 1) * ntiles / 8, nn = n_hi - n_lo;
  if (nn == 0) return;
  const int m_unit = jb / nn;
  const int n_tile = n_lo + jb % nn;

  int e = 0;
  int64_t row0;
  int m;
  if (kMode == kModeDense) {
    row0 = (int64_t)m_unit * BM;
    if (row0 >= a.M) return;
    m = (int)(a.M - row0 < BM ? a.M - row0 : BM);
  } else {
    int loc;
    find_unit<BM>(a.offsets, a.E, m_unit, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e] + (int64_t)loc * BM;
    m = min(BM, a.offsets[e + 1] - (int)row0);
  }
  const int64_t K = a.K;
  const int64_t wrow = K / 2, srow = K / 32;
  const int64_t arow = kActFP4 ? K / 2 : K;

  // activation row (rows past m read row 0 of the tile's first source; never stored)
  auto a_src_row = [&](int r) -> int64_t {
    if (r >= m) r = 0;
    return (kMode == kModeFC1) ? (int64_t)(a.sorted_pair[row0 + r] / a.topk) : row0 + r;
  };
  auto b_row = [&](int r) -> int64_t {
    if (kMode == kModeFC1) return (r < BN / 2 ? 0 : a.I - BN / 2) + (int64_t)n_tile * (BN / 2) + r;
    return (int64_t)n_tile * BN + r;
  };

  // per-lane global sources of this wave's DMA instructions (stage 0)
  const uint8_t* pa[C::IA];
  const uint8_t* pb[C::IB];
  const uint8_t* psa[C::ISA];
  const uint8_t* psb[C::ISB];
#pragma unroll
  for (int q = 0; q < C::IA; ++q) {
    const int chunk = (wave * C::IA + q) * 64 + lane;  // LDS chunk this lane fills
    const int r = chunk / C::CA, pc = chunk % C::CA;
    pa[q] = a.act + a_src_row(r) * arow + 16 * (pc ^ swz<C::CA>(r));
  }
#pragma unroll
  for (int q = 0; q < C::IB; ++q) {
    const int chunk = (wave * C::IB + q) * 64 + lane;
    const int r = chunk / C::CB, pc = chunk % C::CB;
    pb[q] = a.w + ((int64_t)e * a.N + b_row(r)) * wrow + 16 * (pc ^ swz<C::CB>(r));
  }
#pragma unroll
  for (int q = 0; q < C::ISA; ++q) {
    const int dw = (wave * C::ISA + q) * 64 + lane;  // dword of the A-scale slot
    const int r = dw / (C::SB / 4), part = dw % (C::SB / 4);
    psa[q] = a.act_scale + a_src_row(r) * srow + 4 * part;
  }
#pragma unroll
  for (int q = 0; q < C::ISB; ++q) {
    const int dw = (wave * C::ISB + q) * 64 + lane;
    const int r = dw / (C::SB / 4), part = dw % (C::SB / 4);
    psb[q] = a.w_scale + ((int64_t)e * a.N + b_row(r)) * srow + 4 * part;
  }

  auto issue = [&](T3Slot<kActFP4>& sl, int st) {
    const int64_t oa = (int64_t)st * C::RA, ob = (int64_t)st * C::RB, os = (int64_t)st * C::SB;
#pragma unroll
    for (int q = 0; q < C::IA; ++q)
      dma16_to_lds(pa[q] + oa, &sl.A[(wave * C::IA + q) * 1024]);
#pragma unroll
    for (int q = 0; q < C::IB; ++q)
      dma16_to_lds(pb[q] + ob, &sl.B[(wave * C::IB + q) * 1024]);
#pragma unroll
    for (int q = 0; q < C::ISA; ++q)
      dma4_to_lds(psa[q] + os, &sl.As[(wave * C::ISA + q) * 256]);
#pragma unroll
    for (int q = 0; q < C::ISB; ++q)
      dma4_to_lds(psb[q] + os, &sl.Bs[(wave * C::ISB + q) * 256]);
  };

  v16f acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = v16f{};

  int arow_l[2], brow_l[4];
#pragma unroll
  for (int f = 0; f < 2; ++f) arow_l[f] = 64 * wm + 32 * f + r32;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    if (kMode == kModeFC1) brow_l[f] = (f < 2 ? 0 : BN / 2) + 64 * wn + 32 * (f & 1) + r32;
    else brow_l[f] = 128 * wn + 32 * f + r32;
  }

  auto compute = [&](const T3Slot<kActFP4>& sl) {
    int sa[2], sb[4];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      if (C::SB == 8) sa[f] = *reinterpret_cast<const int*>(&sl.As[arow_l[f] * 8 + 4 * g]);
      else sa[f] = *reinterpret_cast<const uint16_t*>(&sl.As[arow_l[f] * 4 + 2 * g]);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      if (C::SB == 8) sb[f] = *reinterpret_cast<const int*>(&sl.Bs[brow_l[f] * 8 + 4 * g]);
      else sb[f] = *reinterpret_cast<const uint16_t*>(&sl.Bs[brow_l[f] * 4 + 2 * g]);
    }
#pragma unroll
    for (int s = 0; s < C::S; ++s) {
      v8i af[2], bf[4];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int r = arow_l[f];
        const uint8_t* rowp = &sl.A[r * C::RA];
        if (kActFP4) {
          const int c = C::S * g + s;
          const v4i x4 = *reinterpret_cast<const v4i*>(rowp + 16 * (c ^ swz<C::CA>(r)));
          af[f] = v8i{x4[0], x4[1], x4[2], x4[3], 0, 0, 0, 0};
        } else {
          const int c1 = 2 * s + g, c2 = 2 * (C::S + s) + g;
          const v4i lo = *reinterpret_cast<const v4i*>(rowp + 16 * (c1 ^ swz<C::CA>(r)));
          const v4i hi = *reinterpret_cast<const v4i*>(rowp + 16 * (c2 ^ swz<C::CA>(r)));
          af[f] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int r = brow_l[f];
        const int c = C::S * g + s;
        const v4i y4 = *reinterpret_cast<const v4i*>(&sl.B[r * C::RB + 16 * (c ^ swz<C::CB>(r))]);
        bf[f] = v8i{y4[0], y4[1], y4[2], y4[3], 0, 0, 0, 0};
      }
#pragma unroll
      for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 4; ++fn) {
          if (s == 0) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 0>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 1) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 1>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else if (s == 2) acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 2>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
          else acc[fm][fn] = mfma32x32x64<kFA, kFmtFP4, 3>(af[fm], bf[fn], acc[fm][fn], sa[fm], sb[fn]);
        }
    }
  };

  // ring pipeline: at stage st, stages st..st+NS-2 have been issued; wait for st
  // (leaving the later ones in flight), barrier, refill the slot freed by st-1, compute st
  constexpr int NS = C::NS, D = C::D;
  const int nst = NST > 0 ? NST : (int)(K / C::KS);
  // every ring step is a compile-time instance, so each DMA and each LDS read names
  // its slot object (the compiler then keeps the loads of other slots in flight)
  auto slot_of = [&](auto I) -> T3Slot<kActFP4>& {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) {
      return slot0;
    } else if constexpr (i == 1) {
      return slot1;
    } else {
      if constexpr (kActFP4) return slot2;  // the 3rd slot exists for FP4 only
      else return slot0;                    // never reached: FP8 runs a 2-slot ring
    }
  };
  auto step = [&](auto I, int st) {
    constexpr int i = decltype(I)::value;
    constexpr int inext = (i + NS - 1) % NS;
    if (NS == 3 && st + 1 < nst) wait_vmcnt<D>();  // stage st+1 may stay in flight
    else wait_vmcnt<0>();
    lds_barrier();
    if (st + NS - 1 < nst) issue(slot_of(std::integral_constant<int, inext>{}), st + NS - 1);
    compute(slot_of(I));
  };
  issue(slot0, 0);
  if constexpr (NS == 3) {
    if (nst > 1) issue(slot1, 1);
  }
  auto ring_turn = [&](int st0) {
    step(std::integral_constant<int, 0>{}, st0);
    if (st0 + 1 < nst) step(std::integral_constant<int, 1>{}, st0 + 1);
    if constexpr (NS == 3) {
      if (st0 + 2 < nst) step(std::integral_constant<int, 2>{}, st0 + 2);
    }
  };
  if constexpr (NST > 0) {
#pragma unroll
    for (int st0 = 0; st0 < NST; st0 += NS) ring_turn(st0);
  } else {
    for (int st0 = 0; st0 < nst; st0 += NS) ring_turn(st0);
  }
  lds_barrier();  // every wave is done reading the ring; slot0 becomes epilogue staging

  // epilogues, 64-row halves staged in slot0 (the waves with wm == half write)
  uint8_t* stage = slot0.A;
  if (kMode == kModeFC1) {
    float(*hf)[BN / 2 + 4] = reinterpret_cast<float(*)[BN / 2 + 4]>(stage);
    const int64_t i0 = (int64_t)n_tile * (BN / 2);
    const int64_t hrow = kActFP4 ? a.I / 2 : a.I;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rr = 32 * fm + 8 * (v >> 2) + 4 * g + (v & 3);
              hf[rr][64 * wn + 32 * f + r32] = silu_mul(acc[fm][f][v], acc[fm][f + 2][v]);
            }
      }
      __syncthreads();
      const int rr = tid >> 2, blk = tid & 3;  // 64 rows x 4 blocks of 32 = 256 items
      const int lr = 64 * half + rr;
      if (lr < m) {
        const int64_t R = row0 + lr;
        quantize_store32<kActFP4>(&hf[rr][32 * blk], a.h + R * hrow + (i0 + 32 * blk) / (kActFP4 ? 2 : 1),
                                  a.h_scale + R * (a.I / 32) + i0 / 32 + blk);
      }
      __syncthreads();
    }
  } else if (kYBF16) {
    uint16_t(*ob)[BN + 8] = reinterpret_cast<uint16_t(*)[BN + 8]>(stage);
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (wm == half) {
#pragma unroll
        for (int fm = 0; fm < 2; ++fm)
#pragma unroll
          for (int fn = 0; fn < 4; ++fn)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int rr = 32 * fm + 8 * (v >> 2) + 4 * g + (v & 3);
              ob[rr][128 * wn + 32 * fn + r32] = (uint16_t)bf16_round(acc[fm][fn][v]);
            }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < (64 * BN / 8) / 256; ++q) {
        const int idx = tid + 256 * q;
        const int rr = idx >> 5, cc = (idx & 31) * 8;
        const int lr = 64 * half + rr;
        if (lr < m)
          *reinterpret_cast<uint4*>(out + (row0 + lr) * a.N + (int64_t)n_tile * BN + cc) =
              *reinterpret_cast<const uint4*>(&ob[rr][cc]);
      }
      __syncthreads();
    }
  } else {
    float(*of)[BN + 4] = reinterpret_cast<float(*)[BN + 4]>(stage);
    float* out = static_cast<float*>(a.out);
#pragma unroll
    for (int quarter = 0; quarter < 4; ++quarter) {
      if (wm == (quarter >> 1)) {
        const int fm = quarter & 1;
#pragma unroll
        for (int fn = 0; fn < 4; ++fn)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rr = 8 * (v >> 2) + 4 * g + (v & 3);
            of[rr][128 * wn + 32 * fn + r32] = acc[fm][fn][v];
          }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < (32 * BN / 4) / 256; ++q) {
        const int idx = tid + 256 * q;
        const int rr = idx >> 6, cc = (idx & 63) * 4;
        const int lr = 32 * quarter + rr;
        if (lr < m)
          *reinterpret_cast<float4*>(out + (row0 + lr) * a.N + (int64_t)n_tile * BN + cc) =
              *reinterpret_cast<const float4*>(&of[rr][cc]);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
// host launchers

template <bool kActFP4, int kMode, bool kYBF16>
static void launch_stream(const GemmArgs& a, int mt, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 1: gemm_stream_kernel<kActFP4, kMode, kYBF16, 1><<<grid, 256, 0, stream>>>(a); break;
    case 2: gemm_stream_kernel<kActFP4, kMode, kYBF16, 2><<<grid, 256, 0, stream>>>(a); break;
    case 3: gemm_stream_kernel<kActFP4, kMode, kYBF16, 3><<<grid, 256, 0, stream>>>(a); break;
    default: gemm_stream_kernel<kActFP4, kMode, kYBF16, 4><<<grid, 256, 0, stream>>>(a); break;
  }
}

template <int kMode, bool kYBF16>
static void launch_stream_fmt(bool fp4, const GemmArgs& a, int mt, dim3 grid, hipStream_t stream) {
  if (fp4) launch_stream<true, kMode, kYBF16>(a, mt, grid, stream);
  else launch_stream<false, kMode, kYBF16>(a, mt, grid, stream);
}

template <int kMode, bool kYBF16>
static void launch_tile2_fmt(bool fp4, GemmArgs a, int64_t m_units, hipStream_t stream) {
#if MXF_TILE_V1
  // first-generation 128 x 128 kernel (16x16x128 MFMA)
  a.ntiles = (int)(kMode == kModeFC1 ? a.I / 64 : a.N / kBN);
  dim3 g1((unsigned)(a.ntiles * (kMode == kModeDense ? cdiv(a.M, kBM) : cdiv(m_units * t2::BM, kBM) + a.E)));
  if (fp4) gemm_tile_kernel<true, kMode, kYBF16><<<g1, 256, 0, stream>>>(a);
  else gemm_tile_kernel<false, kMode, kYBF16><<<g1, 256, 0, stream>>>(a);
  return;
#endif
#if MXF_TILE_V3
  {
    const int64_t nn3 = cdiv(a.ntiles, 8);
    dim3 g3((unsigned)(8 * nn3 * m_units));
    const int64_t nst = a.K / 256;
    if (fp4) {
      if (nst == 28) gemm_tile3_kernel<true, kMode, kYBF16, 28><<<g3, 256, 0, stream>>>(a);
      else if (nst == 8) gemm_tile3_kernel<true, kMode, kYBF16, 8><<<g3, 256, 0, stream>>>(a);
      else gemm_tile3_kernel<true, kMode, kYBF16, 0><<<g3, 256, 0, stream>>>(a);
    } else {
      if (nst == 28) gemm_tile3_kernel<false, kMode, kYBF16, 28><<<g3, 256, 0, stream>>>(a);
      else if (nst == 8) gemm_tile3_kernel<false, kMode, kYBF16, 8><<<g3, 256, 0, stream>>>(a);
      else gemm_tile3_kernel<false, kMode, kYBF16, 0><<<g3, 256, 0, stream>>>(a);
    }
    return;
  }
#endif
#if MXF_T2_XCD
  // 8 XCDs x (m-units x n-tiles per XCD); blocks past the real work exit at once
  const int64_t nn = cdiv(a.ntiles, 8);
  dim3 grid((unsigned)(8 * nn * m_units));
#else
  dim3 grid((unsigned)(a.ntiles * m_units));
#endif
  if (fp4) gemm_tile2_kernel<true, kMode, kYBF16><<<grid, 256, 0, stream>>>(a);
  else gemm_tile2_kernel<false, kMode, kYBF16><<<grid, 256, 0, stream>>>(a);
}

template <int kMode, bool kYBF16>
static void launch_tile_fmt(bool fp4, const GemmArgs& a, dim3 grid, hipStream_t stream) {
  if (fp4) gemm_tile_kernel<true, kMode, kYBF16><<<grid, 256, 0, stream>>>(a);
  else gemm_tile_kernel<false, kMode, kYBF16><<<grid, 256, 0, stream>>>(a);
}

int launch_dense_gemm(const uint8_t* qa, const uint8_t* qa_scale, bool act_fp4, int64_t M, int64_t N, int64_t K,
                      const uint8_t* w, const uint8_t* w_scale, float* c, hipStream_t stream) {
  if (M == 0) return 0;
  GemmArgs a{};
  a.w = w;
  a.w_scale = w_scale;
  a.K = K;
  a.N = N;
  a.E = 1;
  a.topk = 1;
  const int64_t arow = act_fp4 ? K / 2 : K;
  if (M > 64 && N % t2::BN == 0) {
    a.act = qa;
    a.act_scale = qa_scale;
    a.out = c;
    a.M = M;
    a.ntiles = (int)(N / t2::BN);
    launch_tile2_fmt<kModeDense, false>(act_fp4, a, cdiv(M, t2::BM), stream);
  } else {
    for (int64_t m0 = 0; m0 < M; m0 += 64) {
      const int64_t mm = M - m0 < 64 ? M - m0 : 64;
      a.act = qa + m0 * arow;
      a.act_scale = qa_scale + m0 * (K / 32);
      a.out = c + m0 * N;
      a.M = mm;
      dim3 grid((unsigned)cdiv(N, 64), 1);
      launch_stream_fmt<kModeDense, false>(act_fp4, a, (int)cdiv(mm, 16), grid, stream);
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_grouped_gemm(const uint8_t* q, const uint8_t* q_scale, bool act_fp4, int64_t T, int topk, int64_t H,
                        int64_t I, int E, const int32_t* expert_offsets, const int32_t* sorted_pair,
                        const uint8_t* w1, const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale,
                        uint8_t* h, uint8_t* h_scale, void* y, bool y_bf16, hipStream_t stream) {
  const int64_t R = T * topk;
  if (R == 0) return 0;
  GemmArgs f1{};
  f1.act = q;
  f1.act_scale = q_scale;
  f1.w = w1;
  f1.w_scale = w1_scale;
  f1.offsets = expert_offsets;
  f1.sorted_pair = sorted_pair;
  f1.h = h;
  f1.h_scale = h_scale;
  f1.K = H;
  f1.N = 2 * I;
  f1.I = I;
  f1.topk = topk;
  f1.E = E;
  GemmArgs f2 = f1;
  f2.act = h;
  f2.act_scale = h_scale;
  f2.w = w2;
  f2.w_scale = w2_scale;
  f2.out = y;
  f2.K = I;
  f2.N = H;
  const int64_t slots = R < E ? R : E;
  if (T <= 64) {
    const int mt = (int)cdiv(T, 16);
    launch_stream_fmt<kModeFC1, false>(act_fp4, f1, mt, dim3((unsigned)(I / 32), (unsigned)slots), stream);
    if (y_bf16)
      launch_stream_fmt<kModeFC2, true>(act_fp4, f2, mt, dim3((unsigned)cdiv(H, 64), (unsigned)slots), stream);
    else
      launch_stream_fmt<kModeFC2, false>(act_fp4, f2, mt, dim3((unsigned)cdiv(H, 64), (unsigned)slots), stream);
  } else {
    // upper bound on the 128-row tiles summed over experts: each non-empty expert adds at most one partial tile
    const int64_t mtiles = cdiv(R, t2::BM) + slots;
    f1.ntiles = (int)(I / (t2::BN / 2));
    f2.ntiles = (int)(H / t2::BN);
    launch_tile2_fmt<kModeFC1, false>(act_fp4, f1, mtiles, stream);
    if (y_bf16)
      launch_tile2_fmt<kModeFC2, true>(act_fp4, f2, mtiles, stream);
    else
      launch_tile2_fmt<kModeFC2, false>(act_fp4, f2, mtiles, stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

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
    wp[f] = a.w + ((int64_t)e * a.N + nr) * wrow_bytes + 64 * g;
    sp[f] = a.w_scale + ((int64_t)e * a.N + nr) * srow_bytes + 4 * g;
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
    ap[mt] = a.act + src * arow_bytes;
    asp[mt] = a.act_scale + src * srow_bytes + 4 * g;
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
        const v4i* src = reinterpret_cast<const v4i*>(wp[f] + (int64_t)ss * 256);
#pragma unroll
        for (int s = 0; s < 4; ++s) bq[f][s] = __builtin_nontemporal_load(src + s);
        bs[f] = *reinterpret_cast<const int*>(sp[f] + (int64_t)ss * 16);
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
          const v4i* src = reinterpret_cast<const v4i*>(ap[mt] + (int64_t)ss * 256 + 64 * g);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            v4i x = src[s];
            aq[s] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
          }
        } else {
          const uint8_t* base = ap[mt] + (int64_t)ss * 512 + 128 * (g >> 1) + 16 * (g & 1);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            v4i lo = *reinterpret_cast<const v4i*>(base + 32 * s);
            v4i hi = *reinterpret_cast<const v4i*>(base + 256 + 32 * s);
            aq[s] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
        as = *reinterpret_cast<const int*>(asp[mt] + (int64_t)ss * 16);
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
struct TileSmem {
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
  if (M > 64 && N % kBN == 0) {
    a.act = qa;
    a.act_scale = qa_scale;
    a.out = c;
    a.M = M;
    a.ntiles = (int)(N / kBN);
    dim3 grid((unsigned)(a.ntiles * cdiv(M, kBM)));
    launch_tile_fmt<kModeDense, false>(act_fp4, a, grid, stream);
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
    const int64_t mtiles = cdiv(R, kBM) + slots;
    f1.ntiles = (int)(I / 64);
    f2.ntiles = (int)(H / kBN);
    launch_tile_fmt<kModeFC1, false>(act_fp4, f1, dim3((unsigned)(f1.ntiles * mtiles)), stream);
    if (y_bf16)
      launch_tile_fmt<kModeFC2, true>(act_fp4, f2, dim3((unsigned)(f2.ntiles * mtiles)), stream);
    else
      launch_tile_fmt<kModeFC2, false>(act_fp4, f2, dim3((unsigned)(f2.ntiles * mtiles)), stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

// Weight-streaming MXFP4 GEMM for few rows per expert (decode, small dense M):
// every weight byte is read once, as whole 128-byte lines with non-temporal
// loads, and turned into the 16x16x128 scaled MFMA's lane layout through a small
// per-wave LDS area; the K range is split over the 4 waves of a workgroup and
// reduced through LDS in a fixed order. One workgroup = one expert x 64 weight
// rows (FC1: 32 gate + the 32 matching up rows, so SwiGLU stays local). A dense
// variant for at most 16 rows takes bf16 activations and quantises them in registers
// (gemm_stream_q_kernel: 4 waves, or 8 for a one-launch call of at least 8 super-steps).
#include "gemm_common.hpp"

namespace mxf {

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

// ---------------------------------------------------------------------------------
// Activation quantisation inside the dense GEMM (M <= 16): a lane loads the bf16
// values its MFMA operand holds and encodes them in registers, so the codes never
// leave the compute unit.

// largest bf16 magnitude (as bits) among the 8 bf16 values of x
__device__ __forceinline__ uint32_t bf16_absmax8(v4i x) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = (uint32_t)x[i] & 0x7FFF7FFFu;
    m = max(m, max(u & 0xFFFFu, u >> 16));
  }
  return m;
}

// 16 bf16 values (k order, x0 then x1) -> 16 E4M3 codes (4 words, little-endian k
// order) at scale byte `byte`, by gfx950's scaled FP8 conversion (value / scale, round
// to nearest even on the E4M3 grid, subnormals included). That conversion does not
// saturate, so every value is first clamped to +-448 x scale: with it the codes are
// the saturating ones of the block rule. Blocks with a scale byte below 64 are lifted
// by 2^64 (values and scale alike, exact) so that the scale and the values stay
// normal fp32 numbers.
__device__ __forceinline__ void e4m3_encode16(v4i x0, v4i x1, uint32_t byte, uint32_t (&out)[4]) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const bool lift = byte < 64u;
  const float sc = __uint_as_float((byte + (lift ? 64u : 0u)) << 23);
  const float lim = 448.0f * sc;
  const bool any_lift = __builtin_amdgcn_ballot_w64(lift) != 0;
  const float mul = lift ? 18446744073709551616.0f : 1.0f;
  const uint32_t w[8] = {(uint32_t)x0[0], (uint32_t)x0[1], (uint32_t)x0[2], (uint32_t)x0[3],
                         (uint32_t)x1[0], (uint32_t)x1[1], (uint32_t)x1[2], (uint32_t)x1[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v[4] = {__uint_as_float(w[2 * j] << 16), __uint_as_float(w[2 * j] & 0xFFFF0000u),
                  __uint_as_float(w[2 * j + 1] << 16), __uint_as_float(w[2 * j + 1] & 0xFFFF0000u)};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (any_lift) v[i] *= mul;
      v[i] = __builtin_amdgcn_fmed3f(v[i], -lim, lim);
    }
    v2s o = {0, 0};
#if defined(__HIP_DEVICE_COMPILE__)
    o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, v[0], v[1], sc, false);
    o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, v[2], v[3], sc, true);
#endif
    out[j] = __builtin_bit_cast(uint32_t, o);
  }
}

// One 16-row fragment of a 512-k super-step from bf16 (raw: the 16 16-byte loads of
// the lane, 4 per MFMA step s) to the MFMA operands: aq[s] codes, as the 4 scale bytes
// (byte s = block 4 s + g of the super-step, the lane's own block index). Lane (g, r16):
//   E2M1: raw[4 s .. 4 s + 3] are k 128 s + 32 g + [0, 32): one whole block;
//   E4M3: raw[4 s], raw[4 s + 1] are k 128 s + 16 g + [0, 16) (block 4 s + g / 2) and
//         raw[4 s + 2], raw[4 s + 3] are k 128 s + 64 + 16 g + [0, 16) (block
//         4 s + 2 + g / 2): each block is split between lanes g and g ^ 1 (lane ^ 16),
//         which exchange their half-block amax; the scale byte of block 4 s + g then
//         sits with lane g itself (g = 0: low half, g = 3: high half) or with the
//         partner lane ^ 48 (g = 1 takes g = 2's low-half byte, g = 2 takes g = 1's
//         high-half byte).
// Rows past the GEMM's M (valid false) give zero codes and scales.
template <bool kActFP4>
__device__ __forceinline__ void quantize_fragment(const v4i (&raw)[16], bool valid, v8i (&aq)[4], int& as) {
  const int g = (threadIdx.x & 63) >> 4;
  uint32_t lo_b = 0, hi_b = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (kActFP4) {
      float v[32];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t u = (uint32_t)raw[4 * s + i][j];
          v[8 * i + 2 * j] = __uint_as_float(u << 16);
          v[8 * i + 2 * j + 1] = __uint_as_float(u & 0xFFFF0000u);
        }
      uint32_t out[8];
      const uint32_t byte = quantize_block32<true>(v, out);
      aq[s] = valid ? v8i{(int)out[0], (int)out[1], (int)out[2], (int)out[3], 0, 0, 0, 0} : v8i{};
      lo_b |= byte << (8 * s);
    } else {
      uint32_t mlo = max(bf16_absmax8(raw[4 * s]), bf16_absmax8(raw[4 * s + 1]));
      uint32_t mhi = max(bf16_absmax8(raw[4 * s + 2]), bf16_absmax8(raw[4 * s + 3]));
      mlo = max(mlo, (uint32_t)__shfl_xor((int)mlo, 16));
      mhi = max(mhi, (uint32_t)__shfl_xor((int)mhi, 16));
      const uint32_t blo = scale_byte_from_amax_bits(mlo << 16, kEmaxE4M3);
      const uint32_t bhi = scale_byte_from_amax_bits(mhi << 16, kEmaxE4M3);
      uint32_t lo[4], hi[4];
      e4m3_encode16(raw[4 * s], raw[4 * s + 1], blo, lo);
      e4m3_encode16(raw[4 * s + 2], raw[4 * s + 3], bhi, hi);
      aq[s] = valid ? v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                          (int)hi[3]}
                    : v8i{};
      lo_b |= blo << (8 * s);
      hi_b |= bhi << (8 * s);
    }
    // one step's temporaries at a time (the compiler would otherwise interleave the
    // steps and run out of registers)
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kActFP4) {
    as = valid ? (int)lo_b : 0;
  } else {
    const uint32_t got = (uint32_t)__shfl_xor((int)(g == 2 ? lo_b : hi_b), 48);
    const uint32_t b = g == 0 ? lo_b : g == 3 ? hi_b : got;
    as = valid ? (int)b : 0;
  }
}

// ---------------------------------------------------------------------------------
// weight-streaming kernel (rows per expert <= 16 * MT)
//
// K order inside a 512-k super-step: step s, hardware block hb <-> memory block
// 4 s + hb. An FP4 activation lane (g, r16) then reads its 16 bytes of step s at
// 64 s + 16 g, and an FP8 lane's two 16-byte halves sit at 128 s + 16 g and
// 128 s + 64 + 16 g. The scale of (row, block 4 s + g) is byte
// 4 s + g of the row's 16 scale bytes, so a lane gathers bytes g, 4+g, 8+g and
// 12+g of them into one register (op_sel = s picks byte s).
__device__ __forceinline__ int gather_scales(v4i d, int g) {
  const int sh = 8 * g;
  return (int)((((uint32_t)d[0] >> sh) & 0xFFu) | ((((uint32_t)d[1] >> sh) & 0xFFu) << 8) |
               ((((uint32_t)d[2] >> sh) & 0xFFu) << 16) | ((((uint32_t)d[3] >> sh) & 0xFFu) << 24));
}

// Weight loads read whole 128-byte lines with non-temporal loads (lines read once
// per launch): load instruction s of a 16-row fragment gives lane 8 q + j row
// 8 (s & 1) + q of the fragment and 16-byte block 8 (s >> 1) + ((j + q) & 7) of
// that row's 256-byte super-step chunk. Each wave then moves a fragment through a
// private LDS area into the MFMA lane layout (lane (g, r16): row r16, block
// 4 s + g). Instruction s is stored at s * kStgStride + 16 lane; the stride is
// 128 (mod 256) bytes off for odd s and the rotation by q spreads the 16 rows
// read by a lane group over all 64 banks.
constexpr int kStgStride = 1152;
constexpr int kStgBytes = 4 * kStgStride;

// NB: consecutive 64-row blocks per workgroup (FC2 / dense only), streamed one after
// the other by every wave, so that a wave of a short-K GEMM streams NB super-steps
// kQ: dense only, M <= 16 - a.act holds the bf16 activations [M][K], quantised in registers
// WV: waves per workgroup, splitting the K range between them (4; 8 for the one-launch
// dense GEMM with in-register quantisation, whose single workgroup then streams one
// super-step per wave instead of two after one another)
template <bool kActFP4, int kMode, bool kYBF16, int MT, int NB = 1, bool kQ = false, int WV = 4>
__device__ __forceinline__ void stream_body(const GemmArgs& a) {
  static_assert(NB == 1 || kMode != kModeFC1, "FC1 workgroups own one 64-row block");
  static_assert(!kQ || (kMode == kModeDense && MT == 1 && NB == 1), "in-register quantisation: dense, one fragment");
  static_assert(WV == 4 || (kQ && WV == 8), "four waves, or eight for the in-register dense kernel");
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  // per wave: two fragment staging areas in the loop, then NB x MT x 16 x 64 fp32 partial sums
  constexpr int kWaveBytes = 2 * kStgBytes > NB * MT * 4096 ? 2 * kStgBytes : NB * MT * 4096;
  __shared__ v4i lds[WV][kWaveBytes / 16];
  // wave-uniform values made visible as such (readfirstlane), so that the K range, and
  // with it every buffer load's scalar offset, stays in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;

  int e = 0;
  int64_t row0 = 0;
  int m = 0;
  if (kMode == kModeDense) {
    m = (int)a.M;
  } else {
    int loc;
    find_unit<0>(a.offsets, a.E, a.split, blockIdx.y, e, loc);
    if (e < 0) return;
    row0 = a.offsets[e];
    m = a.offsets[e + 1] - (int)row0;
  }
  const int64_t K = a.K;
  const int64_t wrow_bytes = K / 2, srow_bytes = K / 32;
  const int64_t arow_bytes = kActFP4 ? K / 2 : K;

  // the 4 weight fragments of each of the NB row blocks: rows n0 + roff[nb][f] + [0, 16),
  // read through buffer resources over the workgroup's row span (below 4 GiB,
  // checked on the host)
  int64_t n0, span;
  int roff[NB][4];
  bool fvalid[NB][4];
  if (kMode == kModeFC1) {
    n0 = (int64_t)blockIdx.x * 32;  // gate rows n0 + [0, 32), up rows I + n0 + [0, 32)
    span = a.I + 32;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      roff[0][f] = (f < 2 ? 0 : (int)a.I) + 16 * (f & 1);
      fvalid[0][f] = true;
    }
  } else {
    n0 = (int64_t)blockIdx.x * 64 * NB;
    span = min((int64_t)64 * NB, a.N - n0);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        roff[nb][f] = 64 * nb + 16 * f;
        fvalid[nb][f] = 64 * nb + 16 * f < span;
      }
  }
  // the expert index is workgroup-uniform; readfirstlane lets the compiler see that,
  // so the resources sit in scalar registers (no waterfall loop around each load)
  const int64_t rbase = (int64_t)__builtin_amdgcn_readfirstlane(e) * a.N + n0;
  const buf_rsrc wr = make_rsrc(a.w + rbase * wrow_bytes, (uint32_t)(span * wrow_bytes));
  const buf_rsrc sr = make_rsrc(a.w_scale + rbase * srow_bytes, (uint32_t)(span * srow_bytes));
  const int q = lane >> 3, rot = ((lane & 7) + q) & 7;
  const uint32_t wvoff = (uint32_t)(q * wrow_bytes + 16 * rot);
  const uint32_t svoff = (uint32_t)(r16 * srow_bytes);
  // LDS byte offsets: where this lane's loaded block goes, and where its MFMA operand of step s is
  uint8_t* const stg = reinterpret_cast<uint8_t*>(&lds[wave][0]);
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    rd[s] = (2 * (s >> 1) + (r16 >> 3)) * kStgStride + 128 * (r16 & 7) + 16 * ((4 * s + g - (r16 & 7)) & 7);
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
    if (kQ) ap[mt] = a.act + 2 * (src * K + (kActFP4 ? 32 : 16) * g);  // bf16 bytes
    else ap[mt] = a.act + src * arow_bytes + 16 * g;
    asp[mt] = kQ ? nullptr : a.act_scale + src * srow_bytes;
  }

  v4f acc[NB][MT][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[nb][mt][f] = v4f{0.f, 0.f, 0.f, 0.f};

  // dense with kchunk > 0: grid.y slice s covers super-steps [s kchunk, (s+1) kchunk)
  // and writes its partial sums to slice s of out ([grid.y][M][N])
  const int nss = (int)(K / 512);
  int ss_lo = 0, ss_hi = nss;
  if (kMode == kModeDense && a.kchunk > 0) {
    ss_lo = (int)blockIdx.y * a.kchunk;
    ss_hi = min(nss, ss_lo + a.kchunk);
  }
  const int len = ss_hi - ss_lo;
  const int ss_begin = ss_lo + wave * len / WV, ss_end = ss_lo + (wave + 1) * len / WV;
  for (int ss = ss_begin; ss < ss_end; ++ss) {
    // issue every load of the super-step before any wait: activations and scales
    // (few bytes, mostly L2 hits; rows past m read row 0 and are zeroed below),
    // then the 16 weight lines
    v4i araw[MT][kQ ? 16 : kActFP4 ? 4 : 8], asraw[MT], sraw[4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (kQ) {
        // bf16: 2 bytes per k; E2M1 lanes read k 128 s + 32 g + [0, 32), E4M3 lanes
        // k 128 s + 16 g + [0, 16) and 128 s + 64 + 16 g + [0, 16)
        const uint8_t* src = ap[mt] + (int64_t)ss * 1024;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            araw[mt][4 * s + j] =
                *reinterpret_cast<const v4i*>(src + 256 * s + (kActFP4 ? 16 * j : 16 * (j & 1) + 128 * (j >> 1)));
        continue;
      } else if (kActFP4) {
        const uint8_t* src = ap[mt] + (int64_t)ss * 256;
#pragma unroll
        for (int s = 0; s < 4; ++s) araw[mt][s] = *reinterpret_cast<const v4i*>(src + 64 * s);
      } else {
        const uint8_t* base = ap[mt] + (int64_t)ss * 512;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          araw[mt][2 * s] = *reinterpret_cast<const v4i*>(base + 128 * s);
          araw[mt][2 * s + 1] = *reinterpret_cast<const v4i*>(base + 128 * s + 64);
        }
      }
      asraw[mt] = *reinterpret_cast<const v4i*>(asp[mt] + (int64_t)ss * 16);
    }
    v8i aq[MT][4];
    int as[MT];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      // the next block's loads go out only after this block's LDS work (a compiler
      // memory fence on their offsets): one block's 16 lines in flight per wave
      uint32_t wv = wvoff, sv = svoff;
      if (nb > 0) asm volatile("" : "+v"(wv), "+v"(sv)::"memory");
      // a fragment past N (a ragged last block) re-reads the block's first fragment,
      // so every load stays inside the resource without a branch; its outputs are
      // never stored
      v4i raw[4][4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int ro = fvalid[nb][f] ? roff[nb][f] : 0;
        sraw[f] = buf_load16(sr, sv, (uint32_t)(ro * srow_bytes + ss * 16));
#pragma unroll
        for (int s = 0; s < 4; ++s)
          raw[f][s] = buf_load16_nt(wr, wv + 128 * (s >> 1), (uint32_t)((ro + 8 * (s & 1)) * wrow_bytes + ss * 256));
      }
      if constexpr (kQ) {
        // the bf16 values count as written here, after every weight load has gone out:
        // their unpacking (plain arithmetic, free to move) would otherwise be scheduled
        // first and make the weight loads wait for the activations' round trip
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(araw[0][i]));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (nb == 0 && kQ) {
        if constexpr (kQ) quantize_fragment<kActFP4>(araw[0], avalid[0], aq[0], as[0]);
      } else if (nb == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const v4i z = v4i{0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const v4i lo = avalid[mt] ? araw[mt][kActFP4 ? s : 2 * s] : z;
            const v4i hi = kActFP4 || !avalid[mt] ? z : araw[mt][kActFP4 ? s : 2 * s + 1];
            aq[mt][s] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          as[mt] = avalid[mt] ? gather_scales(asraw[mt], g) : 0;
        }
      }
      int bs[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) bs[f] = gather_scales(sraw[f], g);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        uint8_t* const area = stg + (f & 1) * kStgBytes;
#pragma unroll
        for (int s = 0; s < 4; ++s) *reinterpret_cast<v4i*>(area + s * kStgStride + 16 * lane) = raw[f][s];
        v8i b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v4i x = *reinterpret_cast<const v4i*>(area + rd[s]);
          b[s] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          v4f& c = acc[nb][mt][f];
          c = mfma16x16x128<kFA, kFmtFP4, 0>(aq[mt][0], b[0], c, as[mt], bs[f]);
          c = mfma16x16x128<kFA, kFmtFP4, 1>(aq[mt][1], b[1], c, as[mt], bs[f]);
          c = mfma16x16x128<kFA, kFmtFP4, 2>(aq[mt][2], b[2], c, as[mt], bs[f]);
          c = mfma16x16x128<kFA, kFmtFP4, 3>(aq[mt][3], b[3], c, as[mt], bs[f]);
        }
      }
    }
  }

  void* const out = kMode == kModeDense && a.kchunk > 0
                        ? static_cast<void*>(static_cast<float*>(a.out) + (int64_t)blockIdx.y * a.M * a.N)
                        : a.out;
  // reduce the WV K-slices in a fixed order (deterministic)
  // (each wave writes only its own area, which it alone used in the loop)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          reinterpret_cast<float*>(&lds[wave][0])[((nb * MT + mt) * 16 + f * 4 + v) * 64 + lane] = acc[nb][mt][f][v];
  __syncthreads();
  // one (row block, 16-row fragment) item per wave
  for (int item = wave; item < NB * MT; item += WV) {
    const int nb = item / MT, mt = item % MT;
    float tot[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int idx = item * 16 + f * 4 + v;
        const float* r = reinterpret_cast<const float*>(&lds[0][0]) + idx * 64 + lane;
        constexpr int kW = kWaveBytes / 4;  // floats per wave area
        float t = r[0];
#pragma unroll
        for (int w = 1; w < WV; ++w) t += r[w * kW];
        tot[f][v] = t;
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
            const int64_t n = n0 + 64 * nb + 16 * f + r16;
            if (64 * nb + 16 * f < span) store_out<kYBF16>(out, (row0 + lr) * a.N + n, tot[f][v]);
          }
        }
      }
    }
  }
}

// One 16-row fragment (decode): registers held to three waves per SIMD (168
// VGPRs), with the 16 weight lines of a super-step in flight per wave; measured
// faster than two waves per SIMD with the same loads or three waves with fewer.
template <bool kActFP4, int kMode, bool kYBF16, int NB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) gemm_stream1_kernel(GemmArgs a) {
  stream_body<kActFP4, kMode, kYBF16, 1, NB>(a);
}
template <bool kActFP4, int kMode, bool kYBF16, int MT>
__global__ void __launch_bounds__(256) gemm_stream_kernel(GemmArgs a) {
  stream_body<kActFP4, kMode, kYBF16, MT>(a);
}

// dense GEMM with M <= 16 and bf16 activations quantised in registers
template <bool kActFP4, int WV>
__global__ void __launch_bounds__(64 * WV) gemm_stream_q_kernel(GemmArgs a) {
  stream_body<kActFP4, kModeDense, false, 1, 1, true, WV>(a);
}

void launch_stream_q_gemm(bool act_fp4, const GemmArgs& a, dim3 grid, hipStream_t stream) {
  // one workgroup row over the whole K (no slices) of at least 8 super-steps: eight
  // waves; else four (measured: 16 x 32 x 4096 in 9.75 instead of 11.37 us per call, but
  // 16 x 2048 x 2048, 4 super-steps, in 8.22 instead of 7.39 us)
  const bool wide = grid.y == 1 && a.kchunk == 0 && a.K / 512 >= 8;
  if (act_fp4) {
    if (wide) gemm_stream_q_kernel<true, 8><<<grid, 512, 0, stream>>>(a);
    else gemm_stream_q_kernel<true, 4><<<grid, 256, 0, stream>>>(a);
  } else {
    if (wide) gemm_stream_q_kernel<false, 8><<<grid, 512, 0, stream>>>(a);
    else gemm_stream_q_kernel<false, 4><<<grid, 256, 0, stream>>>(a);
  }
}

// decode FC2 (K = I, a few super-steps): two 64-row blocks per workgroup, measured
// faster than one (0.168 -> 0.163 ms for the 8-token layer's grouped GEMM)
constexpr int kStreamFc2Blocks = 2;

template <bool kActFP4, int kMode, bool kYBF16>
static void launch_stream_mt(const GemmArgs& a, int mt, dim3 grid, hipStream_t stream) {
  switch (mt) {
    case 1:
      if constexpr (kMode == kModeFC2 && kStreamFc2Blocks == 2) {
        // two 64-row blocks per workgroup (K = I is short: one super-step per wave per block)
        grid.x = (unsigned)cdiv(a.N, 128);
        gemm_stream1_kernel<kActFP4, kMode, kYBF16, 2><<<grid, 256, 0, stream>>>(a);
      } else {
        gemm_stream1_kernel<kActFP4, kMode, kYBF16, 1><<<grid, 256, 0, stream>>>(a);
      }
      break;
    case 2: gemm_stream_kernel<kActFP4, kMode, kYBF16, 2><<<grid, 256, 0, stream>>>(a); break;
    case 3: gemm_stream_kernel<kActFP4, kMode, kYBF16, 3><<<grid, 256, 0, stream>>>(a); break;
    default: gemm_stream_kernel<kActFP4, kMode, kYBF16, 4><<<grid, 256, 0, stream>>>(a); break;
  }
}

template <bool kActFP4>
static void launch_stream_fmt(int mode, bool y_bf16, const GemmArgs& a, int mt, dim3 grid, hipStream_t stream) {
  if (mode == kModeFC1) launch_stream_mt<kActFP4, kModeFC1, false>(a, mt, grid, stream);
  else if (mode == kModeDense) launch_stream_mt<kActFP4, kModeDense, false>(a, mt, grid, stream);
  else if (y_bf16) launch_stream_mt<kActFP4, kModeFC2, true>(a, mt, grid, stream);
  else launch_stream_mt<kActFP4, kModeFC2, false>(a, mt, grid, stream);
}

__global__ void __launch_bounds__(256) reduce_partials_kernel(const float4* __restrict__ part, int S, int64_t n4,
                                                              float4* __restrict__ c) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float4 acc = part[i];
  for (int s = 1; s < S; ++s) {
    const float4 p = part[(int64_t)s * n4 + i];
    acc.x += p.x;
    acc.y += p.y;
    acc.z += p.z;
    acc.w += p.w;
  }
  c[i] = acc;
}

void launch_reduce_partials(const float* part, int S, int64_t n, float* c, hipStream_t stream) {
  const int64_t n4 = n / 4;
  reduce_partials_kernel<<<(unsigned)cdiv(n4, 256), 256, 0, stream>>>(reinterpret_cast<const float4*>(part), S, n4,
                                                                     reinterpret_cast<float4*>(c));
}

void launch_stream_gemm(int mode, bool y_bf16, bool act_fp4, const GemmArgs& a, int mt, dim3 grid,
                        hipStream_t stream) {
  if (act_fp4) launch_stream_fmt<true>(mode, y_bf16, a, mt, grid, stream);
  else launch_stream_fmt<false>(mode, y_bf16, a, mt, grid, stream);
}

}  // namespace mxf

// The epilogue shared by the 256 x 256 LDS-ring kernels (gemm_wide.hip: E2M1
// activations; gemm_f8ring.hip: E4M3 activations). Both run 8 waves of 64 x 128 on
// the 32x32x64 scaled MFMA with the weight fragment as the first operand, so the
// accumulators of a wave have the same layout in both.
#pragma once

#include "gemm_common.hpp"

namespace mxf {

// LDS bytes the epilogue stages through (FC2 / dense): 8 waves x 8 KB (bf16) or
// 8 x 4352 B (fp32)
constexpr int kTile256Staging = 8 * 8192;

// Blocks of the launch: dense, XCD x walks nn <= ceil(ntiles / 8) n-tiles for each of
// the m_units row units; grouped, XCD x runs items [x T / 8, (x + 1) T / 8) of the
// T = units x ntiles / ntg items (units <= m_units), so ceil(m_units ntiles / ntg / 8)
// blocks per XCD cover them. Blocks past their XCD's range exit at once, but each
// still waits for a whole compute unit (the ring takes all of its LDS), so the grid
// follows the n-tiles per workgroup.
inline dim3 tile256_grid(int mode, const GemmArgs& a, int64_t m_units, int ntg) {
  const int64_t per_xcd = mode == kModeDense ? cdiv(a.ntiles, 8) * m_units : cdiv(m_units * (a.ntiles / ntg), 8);
  return dim3((unsigned)(8 * per_xcd));
}

// Epilogue of one 256 x 256 tile, straight from the accumulators (FC1 without LDS). The
// MFMAs take the weight fragment as their first operand, so acc[fm][fn][v] of
// lane l is token row 64 wm + 32 fm + l % 32 and output column c(fn) + 8 (v / 4)
// + 4 (l / 32) + v % 4: every lane holds runs of 4 consecutive columns of one row.
// FC1: h = silu(gate) * up, requantised to E2M1 (kHFP4) or E4M3 per 32 I-columns - a
// block is one fragment's 32 columns of one row, held half by lane l and half by
// lane l ^ 32;
// FC2 / dense: y or c in bf16 or fp32 through LDS - bf16 a whole fragment (32 rows)
// at a time in the wave's 8 KB of the slot, fp32 8 rows at a time in a 4352-byte
// region (8- or 16-byte runs in, 16-byte row pieces out, so each store instruction
// writes whole 256- or 512-byte row segments).
template <int kMode, bool kYBF16, bool kHFP4>
__device__ __forceinline__ void tile256_epilogue(const GemmArgs& a, const v16f (&acc)[2][4], uint8_t* slot,
                                                 int n_tile, int64_t row0, int m) {
  constexpr int BN = 256, STG = 4352;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, g = lane >> 5,
            r32 = lane & 31;
  uint8_t* const stg = slot + wave * STG;
  const int wm = wave >> 1, wn = wave & 1;
  if (64 * wm >= m) return;
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    const int lr = 64 * wm + 32 * fm + r32;
    const bool ok = lr < m;
    const int64_t Rw = row0 + lr;
    if (kMode == kModeFC1 && !kHFP4) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {  // gate fragment f, up fragment f + 2: I-columns icol + [0, 32)
        float h[16];
        float amf = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          h[v] = silu_mul(acc[fm][f][v], acc[fm][f + 2][v]);
          amf = fmaxf(amf, fabsf(h[v]));
        }
        uint32_t amax = __float_as_uint(amf);
        amax = max(amax, lane_xor32(amax));
        const uint32_t byte = scale_byte_from_amax_bits(amax, kEmaxE4M3);
        const float inv = inv_scale_from_byte(byte);
        uint32_t c[4];  // c[j]: the E4M3 codes of this lane's column run j (columns 8 j + 4 g .. + 3)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          c[j] = e4m3_code(h[4 * j], inv) | (e4m3_code(h[4 * j + 1], inv) << 8) |
                 (e4m3_code(h[4 * j + 2], inv) << 16) | (e4m3_code(h[4 * j + 3], inv) << 24);
        // the block's 32 bytes: lane g = 0 writes columns 0..15 (its runs 0, 1 and the
        // partner's), lane g = 1 columns 16..31 (the partner's runs 2, 3 and its own)
        const uint32_t p0 = lane_xor32(g ? c[0] : c[2]), p1 = lane_xor32(g ? c[1] : c[3]);
        if (ok) {
          const int64_t icol = (int64_t)n_tile * (BN / 2) + 64 * wn + 32 * f;
          const uint4 d = g ? make_uint4(p0, c[2], p1, c[3]) : make_uint4(c[0], p0, c[1], p1);
          *reinterpret_cast<uint4*>(a.h + Rw * a.I + icol + 16 * g) = d;
          if (g == 0) a.h_scale[Rw * (a.I / 32) + icol / 32] = (uint8_t)byte;
        }
      }
    } else if (kMode == kModeFC1) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {  // gate fragment f, up fragment f + 2: I-columns icol + [0, 32)
        float h[16];
        float amf = 0.0f;  // max |h| (finite, non-negative: the float order is the bit order)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          h[v] = silu_mul(acc[fm][f][v], acc[fm][f + 2][v]);
          amf = fmaxf(amf, fabsf(h[v]));
        }
        uint32_t amax = __float_as_uint(amf);
        amax = max(amax, lane_xor32(amax));
        const uint32_t byte = scale_byte_from_amax_bits(amax, kEmaxE2M1);
        // E2M1 codes by the hardware conversion (equal to e2m1_code); blocks with a
        // scale byte below 64 are lifted by 2^64 (values and scale alike, exact) as in
        // quantize_block32 - a case real data hardly reaches, so the multiplications
        // run only when some lane of the wave needs them
        const bool lift = byte < 64u;
        const float sc = __uint_as_float((byte + (lift ? 64u : 0u)) << 23);
        if (__builtin_amdgcn_ballot_w64(lift) != 0) {
          const float mul = lift ? 18446744073709551616.0f : 1.0f;
#pragma unroll
          for (int v = 0; v < 16; ++v) h[v] *= mul;
        }
        uint32_t c[2];  // bytes 2 j, 2 j + 1 of c[j / 2 ... ]: the 4 codes of column run j
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float* x = &h[8 * q];
          uint32_t w = 0;
#if defined(__HIP_DEVICE_COMPILE__)
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], sc, 0);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], sc, 1);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], sc, 2);
          w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], sc, 3);
#endif
          c[q] = w;
        }
        const uint32_t p0 = lane_xor32(c[0]), p1 = lane_xor32(c[1]);
        // the block's 16 bytes: 2-byte runs in column order, lane g = 0's run j, then lane 1's
        if (g == 0 && ok) {
          const int64_t icol = (int64_t)n_tile * (BN / 2) + 64 * wn + 32 * f;
          const uint4 d = make_uint4((c[0] & 0xFFFFu) | (p0 << 16), (c[0] >> 16) | (p0 & 0xFFFF0000u),
                                     (c[1] & 0xFFFFu) | (p1 << 16), (c[1] >> 16) | (p1 & 0xFFFF0000u));
          *reinterpret_cast<uint4*>(a.h + Rw * (a.I / 2) + icol / 2) = d;
          a.h_scale[Rw * (a.I / 32) + icol / 32] = (uint8_t)byte;
        }
      }
    } else if (kYBF16) {
      // the fragment's 32 rows x 128 columns at once in the wave's 8 KB of slot 1:
      // row r at 256 r, 16-byte piece p at piece p ^ (r % 16), and its two 8-byte
      // halves swapped for r >= 16, so that the 8-byte writes (32 rows of one piece
      // per half-wave) and the 16-byte reads (one row per 16 lanes) both spread over
      // all 64 banks
      uint8_t* const ob = slot + wave * 8192;
      uint16_t* out = static_cast<uint16_t*>(a.out);
      const int64_t col0 = (int64_t)n_tile * BN + 128 * wn;
      const int hs = (r32 >> 4) & 1;
#pragma unroll
      for (int fn = 0; fn < 4; ++fn)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint2 d;
          d.x = bf16x2_bits(acc[fm][fn][4 * j], acc[fm][fn][4 * j + 1]);
          d.y = bf16x2_bits(acc[fm][fn][4 * j + 2], acc[fm][fn][4 * j + 3]);
          *reinterpret_cast<uint2*>(ob + 256 * r32 + 16 * ((4 * fn + j) ^ (r32 & 15)) + 8 * (g ^ hs)) = d;
        }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int k = 0; k < 8; ++k) {  // 32 rows x 16 pieces of 16 bytes
        const int idx = lane + 64 * k;
        const int rr = idx >> 4, c = idx & 15;
        const int lrow = 64 * wm + 32 * fm + rr;
        v4i v = *reinterpret_cast<const v4i*>(ob + 256 * rr + 16 * (c ^ (rr & 15)));
        if (rr & 16) v = v4i{v[2], v[3], v[0], v[1]};
        if (lrow < m)  // y is read once, by the combine: non-temporal stores
          __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(out + (row0 + lrow) * a.N + col0 + 8 * c));
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    } else {
      float(*of)[132] = reinterpret_cast<float(*)[132]>(stg);  // 8 x 132 x 4 = 4224 bytes
      float* out = static_cast<float*>(a.out);
      const int64_t col0 = (int64_t)n_tile * BN + 128 * wn;
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {  // rows r32 in [8 hh, 8 hh + 8)
        if ((r32 >> 3) == hh) {
#pragma unroll
          for (int fn = 0; fn < 4; ++fn)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              *reinterpret_cast<float4*>(&of[r32 & 7][32 * fn + 8 * j + 4 * g]) =
                  make_float4(acc[fm][fn][4 * j], acc[fm][fn][4 * j + 1], acc[fm][fn][4 * j + 2], acc[fm][fn][4 * j + 3]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // 8 rows x 128 columns = 256 pieces of 16 bytes
          const int idx = lane + 64 * j;
          const int rr = idx >> 5, c4 = idx & 31;
          const int lrow = 64 * wm + 32 * fm + 8 * hh + rr;
          if (lrow < m)
            __builtin_nontemporal_store(*reinterpret_cast<const v4i*>(&of[rr][4 * c4]),
                                        reinterpret_cast<v4i*>(out + (row0 + lrow) * a.N + col0 + 4 * c4));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
  }
}

}  // namespace mxf

// FC2 and the gate-weighted combine in one kernel, for decode-sized batches
// (at most 64 tokens):
//   out[t][n] = sum_j gates[t][j] * y[t][j][n],  y[t][j] = h_hat[row(t, j)] . W2_hat[e(t, j)]^T,
// the sum over the slots j = 0, 1, ... in that order, in fp32; y never leaves the chip.
//
// The point is removing the data movement between the two steps rather than making
// either faster (page "【DeepSeek V4】Triton FP4 优化实战", its closing lessons; the
// combine half of MoE dispatch/combine, page "Domestic GPUs are awesome! ...
// DeepSeek-V4"). Token-major: a workgroup owns one token and 16 output columns and
// has one wave per slot j. Wave j streams the 16 W2 rows of those columns of the
// expert e(t, j) over the whole contraction (whole 128-byte lines, moved through a
// private LDS area into the 16x16x128 lane layout, as the weight-streaming GEMM
// does) and multiplies them with the one h row of the pair; the k partial rows meet
// in LDS and the workgroup's first 16 threads add them in slot order. Every wave
// issues all its loads of up to 4 super-steps (16 KB of weights at I = 2048) before
// the first wait, and the grid has T * H / 16 workgroups, so many loads are in
// flight per compute unit. The pair's h row and the weight rows' scale bytes go
// through LDS (one coalesced load each), which keeps them out of the registers. An
// expert picked by several tokens is read once per token; the workgroups of one
// column block run on one XCD back to back (blocks are dealt to the 8 XCDs in turn),
// so the repeats come from that XCD's L2 rather than HBM even with non-temporal
// loads (measured: the kernel fetches as many bytes as the unfused FC2). Forcing
// five waves per SIMD (96 registers) measured slower: the E4M3 form then spills.
// Deterministic: no atomics, fixed summation order, no workspace.
#include "gemm_common.hpp"

namespace mxf {

namespace fc2c {
constexpr int kStgStride = 1152;  // bytes between the 4 load instructions' staging rows
constexpr int kMaxK = 8;
constexpr int kCH = 4;  // super-steps whose loads are issued together (a power of two)
}  // namespace fc2c

struct Fc2cArgs {
  const uint8_t* h;         // [R][I] E4M3 or [R][I/2] E2M1, rows in the permuted order
  const uint8_t* h_scale;   // [R][I/32]
  const uint8_t* w2;        // [E][H][I/2]
  const uint8_t* w2_scale;  // [E][H][I/32]
  const int32_t* topk_ids;  // [T][topk]
  const int32_t* pair_row;  // [T * topk]: permuted row of pair t * topk + j
  const float* gates;       // [T][topk]
  void* out;                // [T][H] bf16 or fp32
  int64_t T, H, I;
  int topk, out_bf16;
};

// LDS bytes per wave: the weight staging area, then kCH super-steps of the h row and
// their 16 scale bytes each, then the 16 NB weight rows' scale bytes of kCH super-steps
__host__ __device__ constexpr int fc2c_wave_bytes(bool act_fp4, int nb) {
  return 4 * fc2c::kStgStride + fc2c::kCH * (act_fp4 ? 256 : 512) + 16 * fc2c::kCH + 16 * nb * 16 * fc2c::kCH;
}

// bytes g, 4 + g, 8 + g, 12 + g of a row's 16 scale bytes of one 512-k super-step:
// the scales of blocks 4 s + g, s = 0..3, one per byte (op_sel = s picks byte s)
__device__ __forceinline__ int fc2c_scales(v4i d, int g) {
  const int sh = 8 * g;
  return (int)((((uint32_t)d[0] >> sh) & 0xFFu) | ((((uint32_t)d[1] >> sh) & 0xFFu) << 8) |
               ((((uint32_t)d[2] >> sh) & 0xFFu) << 16) | ((((uint32_t)d[3] >> sh) & 0xFFu) << 24));
}

// NB: 16-column blocks per workgroup (each wave streams NB x 16 weight rows)
template <bool kActFP4, int NB>
__global__ void __launch_bounds__(64 * fc2c::kMaxK) fc2_combine_kernel(Fc2cArgs a) {
  using namespace fc2c;
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  constexpr int kSS = kActFP4 ? 256 : 512;  // activation bytes of one 512-k super-step
  constexpr int kW = fc2c_wave_bytes(kActFP4, NB);
  // LDS (sized for topk waves at launch): per wave a weight staging area, the h chunk
  // with its scales and the weight scales, then the k x 16 NB partial rows
  extern __shared__ v4i fc2c_lds[];
  // workgroup -> (column block, token): the blocks on XCD x (block index % 8 == x) take
  // a contiguous range of the grid, column block by column block
  const int64_t G = a.T * (a.H / (16 * NB));
  const int64_t per = (G + 7) / 8;
  const int64_t L = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (L >= G) return;  // the whole workgroup (before any barrier)
  const int64_t cb = L / a.T;
  const int t = (int)(L % a.T);
  const int64_t n0 = cb * 16 * NB;
  const int j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the slot of this wave
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int p = t * a.topk + j;
  const int e = __builtin_amdgcn_readfirstlane(a.topk_ids[p]);
  const int hr = __builtin_amdgcn_readfirstlane(a.pair_row[p]);
  const int64_t K = a.I, wrow = K / 2, srow = K / 32, arow = kActFP4 ? K / 2 : K;
  const int64_t R = a.T * a.topk;
  const int nss = (int)(K / 512);
  uint8_t* const stg = reinterpret_cast<uint8_t*>(fc2c_lds) + j * kW;
  uint8_t* const act = stg + 4 * kStgStride;
  uint8_t* const wsc = act + kCH * kSS + 16 * kCH;  // [16 NB rows][kCH super-steps][16 bytes]
  float(*ylds)[16 * NB] = reinterpret_cast<float(*)[16 * NB]>(reinterpret_cast<uint8_t*>(fc2c_lds) + a.topk * kW);
  // load instruction s gives lane 8 q + i row 8 (s & 1) + q and 16-byte block
  // 8 (s >> 1) + ((i + q) & 7) of the row's 256-byte super-step chunk; the lane's
  // MFMA operand of step s (row r16, block 4 s + g) is then read back at rd[s]
  const int q = lane >> 3, rot = ((lane & 7) + q) & 7;
  const uint32_t wvoff = (uint32_t)(q * wrow + 16 * rot);
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    rd[s] = (2 * (s >> 1) + (r16 >> 3)) * kStgStride + 128 * (r16 & 7) + 16 * ((4 * s + g - (r16 & 7)) & 7);
  // the expert's W2 rows n0 .. n0 + 16 NB - 1 (one expert's codes stay below 4 GiB:
  // checked on the host), and all of h (R * I bytes, below 4 GiB as R <= 512):
  // range-checked reads
  const int64_t rbase = (int64_t)e * a.H + n0;
  const buf_rsrc wr = make_rsrc(a.w2 + rbase * wrow, (uint32_t)(16 * NB * wrow));
  const buf_rsrc sr = make_rsrc(a.w2_scale + rbase * srow, (uint32_t)(16 * NB * srow));
  const buf_rsrc hrs = make_rsrc(a.h, (uint32_t)(R * arow));
  const buf_rsrc hss = make_rsrc(a.h_scale, (uint32_t)(R * srow));
  // the pair's h row is the A operand's row 0 (lanes with r16 == 0); its other 15 rows are zero
  const bool arow0 = r16 == 0;

  v4f acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int ss0 = 0; ss0 < nss; ss0 += kCH) {
    // the pair's h row for kCH super-steps first (L2-resident, so it arrives before the
    // weights and waiting for it does not wait for them): kCH * kSS bytes, 16 or 32 per
    // lane, plus 16 scale bytes per super-step on lanes 0 .. kCH-1. Bytes past the row
    // (a partial last chunk) belong to steps whose products are zeroed below.
    const uint32_t abase = (uint32_t)(hr * arow + (int64_t)ss0 * kSS);
    const v4i a0 = buf_load16(hrs, abase + (kActFP4 ? 16 : 32) * lane, 0);
    const v4i a1 = kActFP4 ? v4i{0, 0, 0, 0} : buf_load16(hrs, abase + 32 * lane + 16, 0);
    const v4i asc = buf_load16(hss, (uint32_t)(hr * srow + (int64_t)ss0 * 16 + 16 * (lane & (kCH - 1))), 0);
    // the weight rows' scale bytes of kCH super-steps: load i of lane l takes row
    // 16 i + l / kCH, super-step ss0 + l % kCH (16 bytes); then every weight load of
    // kCH super-steps before the first wait (a super-step past the end re-reads the
    // last one; its products are zeroed)
    const int wss = min(ss0 + lane % kCH, nss - 1);
    v4i wsraw[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wsraw[nb] = buf_load16(sr, (uint32_t)((16 * nb + lane / kCH) * srow + wss * 16), 0);
    v4i raw[NB][kCH][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int c = 0; c < kCH; ++c) {
        const int ss = min(ss0 + c, nss - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          raw[nb][c][s] = buf_load16_nt(wr, wvoff + 128 * (s >> 1),
                                        (uint32_t)((16 * nb + 8 * (s & 1)) * wrow + ss * 256));
      }
    __builtin_amdgcn_sched_barrier(0);
    if (kActFP4) {
      *reinterpret_cast<v4i*>(act + 16 * lane) = a0;
    } else {
      *reinterpret_cast<v4i*>(act + 32 * lane) = a0;
      *reinterpret_cast<v4i*>(act + 32 * lane + 16) = a1;
    }
    if (lane < kCH) *reinterpret_cast<v4i*>(act + kCH * kSS + 16 * lane) = asc;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<v4i*>(wsc + 1024 * nb + 16 * lane) = wsraw[nb];
#pragma unroll
    for (int c = 0; c < kCH; ++c) {
      const bool live = ss0 + c < nss;
      const v4i asr = *reinterpret_cast<const v4i*>(act + kCH * kSS + 16 * c);
      const int as = fc2c_scales(asr, g);
      const bool use = live && arow0;
      v8i av[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v4i z = v4i{0, 0, 0, 0};
        // lane (g, 0) of step s: bytes 64 s + 16 g (E2M1), or 128 s + 16 g and 128 s + 64 + 16 g (E4M3)
        const uint8_t* src = act + c * kSS + (kActFP4 ? 64 : 128) * s + 16 * g;
        const v4i lo4 = *reinterpret_cast<const v4i*>(src);
        const v4i hi4 = kActFP4 ? z : *reinterpret_cast<const v4i*>(src + 64);
        const v4i l = use ? lo4 : z, hgh = use ? hi4 : z;
        av[s] = v8i{l[0], l[1], l[2], l[3], hgh[0], hgh[1], hgh[2], hgh[3]};
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) *reinterpret_cast<v4i*>(stg + s * kStgStride + 16 * lane) = raw[nb][c][s];
        v8i b[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v4i x = *reinterpret_cast<const v4i*>(stg + rd[s]);
          b[s] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
        }
        const v4i bsr = *reinterpret_cast<const v4i*>(wsc + 1024 * nb + 16 * (kCH * r16 + c));
        const int bs = fc2c_scales(bsr, g);
        acc[nb] = mfma16x16x128<kFA, kFmtFP4, 0>(av[0], b[0], acc[nb], as, bs);
        acc[nb] = mfma16x16x128<kFA, kFmtFP4, 1>(av[1], b[1], acc[nb], as, bs);
        acc[nb] = mfma16x16x128<kFA, kFmtFP4, 2>(av[2], b[2], acc[nb], as, bs);
        acc[nb] = mfma16x16x128<kFA, kFmtFP4, 3>(av[3], b[3], acc[nb], as, bs);
      }
    }
  }
  // acc[nb][0] of lanes 0..15 = y[t][j][n0 + 16 nb + lane] (row 0 of the result)
  if (lane < 16) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ylds[j][16 * nb + lane] = acc[nb][0];
  }
  __syncthreads();
  // out[t][n0 + c] = sum_j gates[t][j] * y[t][j][c] over j = 0, 1, ... (fp32 fused multiply-adds)
  if (threadIdx.x < 16 * NB) {
    const int c = threadIdx.x;
    float s = 0.0f;
    for (int jj = 0; jj < a.topk; ++jj) s = fmaf(a.gates[t * a.topk + jj], ylds[jj][c], s);
    const int64_t o = (int64_t)t * a.H + n0 + c;
    if (a.out_bf16) static_cast<uint16_t*>(a.out)[o] = (uint16_t)bf16_round(s);
    else static_cast<float*>(a.out)[o] = s;
  }
}

int launch_fc2_combine(const uint8_t* h, const uint8_t* h_scale, bool act_fp4, int64_t T, int topk, int64_t H,
                       int64_t I, const int32_t* topk_ids, const int32_t* pair_row, const float* gates,
                       const uint8_t* w2, const uint8_t* w2_scale, void* out, bool out_bf16, hipStream_t stream) {
  // one 16-column block per workgroup: two (32 KB per wave in flight, the h row read
  // once for both) measured slower at the 8-token decode layer, 168.6 against 166.0 us
  // for both FCs, as their register use halves the waves per SIMD
  constexpr int NB = 1;
  if (T <= 0) return 0;
  if (topk < 1 || topk > fc2c::kMaxK || H % (16 * NB) != 0 || I % 512 != 0) return -1;
  const Fc2cArgs a{h, h_scale, w2, w2_scale, topk_ids, pair_row, gates, out, T, H, I, topk, out_bf16 ? 1 : 0};
  const int64_t G = T * (H / (16 * NB));
  const dim3 grid((unsigned)(8 * cdiv(G, 8)));
  const dim3 block((unsigned)(64 * topk));
  const size_t lds = (size_t)topk * (fc2c_wave_bytes(act_fp4, NB) + 16 * NB * sizeof(float));
  if (act_fp4) fc2_combine_kernel<true, NB><<<grid, block, lds, stream>>>(a);
  else fc2_combine_kernel<false, NB><<<grid, block, lds, stream>>>(a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

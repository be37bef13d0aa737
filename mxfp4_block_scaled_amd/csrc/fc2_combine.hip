// FC2 and the gate-weighted combine in one kernel, for decode-sized batches
// (at most 64 tokens):
//   out[t][n] = sum_j gates[t][j] * y[t][j][n],  y[t][j] = h_hat[row(t, j)] . W2_hat[e(t, j)]^T,
// the sum over the slots j = 0, 1, ... in that order, in fp32; y never leaves the chip.
//
// The point is removing the data movement between the two steps rather than making
// either faster (page "【DeepSeek V4】Triton FP4 优化实战", its closing lessons; the
// combine half of MoE dispatch/combine, page "Domestic GPUs are awesome! ...
// DeepSeek-V4"). A workgroup owns 16 output columns of every token, so every
// contribution to its part of the output is computed inside it. Its 4 waves share
// out the touched experts (the k-th non-empty expert goes to wave k % 4); a wave
// streams its expert's 16 W2 rows of those columns as whole 128-byte lines with
// non-temporal loads, moves them through a private LDS area into the 16x16x128 lane
// layout (as the weight-streaming GEMM does) and multiplies them with the expert's h
// rows. A (token, slot) pair belongs to exactly one expert, so each y entry is
// written once, in fp32, into an LDS table y[pair][16 columns]; after one barrier
// each thread sums one token's slots for one column in slot order and stores the
// result. Deterministic, no atomics, no workspace: H / 16 workgroups (448 at
// H = 7168), each reading its columns of the touched experts once.
#include "gemm_common.hpp"

namespace mxf {

namespace fc2c {
constexpr int kStgStride = 1152;  // bytes between the 4 load instructions' staging rows
constexpr int kMaxPairs = 512;    // T * topk (T <= 64, topk <= 8)
}  // namespace fc2c

struct Fc2cArgs {
  const uint8_t* h;         // [R][I] E4M3 or [R][I/2] E2M1, rows in the permuted order
  const uint8_t* h_scale;   // [R][I/32]
  const uint8_t* w2;        // [E][H][I/2]
  const uint8_t* w2_scale;  // [E][H][I/32]
  const int32_t* offsets;   // [E+1]
  const int32_t* sorted_pair;
  const float* gates;       // [T][topk]
  void* out;                // [T][H] bf16 or fp32
  int64_t T, H, I;
  int topk, E;
  int out_bf16;
};

// bytes g, 4 + g, 8 + g, 12 + g of a row's 16 scale bytes of one 512-k super-step:
// the scales of blocks 4 s + g, s = 0..3, one per byte (op_sel = s picks byte s)
__device__ __forceinline__ int fc2c_scales(v4i d, int g) {
  const int sh = 8 * g;
  return (int)((((uint32_t)d[0] >> sh) & 0xFFu) | ((((uint32_t)d[1] >> sh) & 0xFFu) << 8) |
               ((((uint32_t)d[2] >> sh) & 0xFFu) << 16) | ((((uint32_t)d[3] >> sh) & 0xFFu) << 24));
}

// CH: 512-k super-steps whose weight loads are all issued before the first is used;
// DA: super-steps of activations in flight ahead of the one being multiplied
template <bool kActFP4, int CH, int DA>
__global__ void __launch_bounds__(256) fc2_combine_kernel(Fc2cArgs a) {
  using namespace fc2c;
  constexpr int kFA = kActFP4 ? kFmtFP4 : kFmtFP8;
  constexpr int kAV = kActFP4 ? 4 : 8;  // 16-byte activation loads per super-step
  __shared__ float ytab[kMaxPairs][16];
  __shared__ v4i stg_all[4][4 * kStgStride / 16];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t K = a.I, wrow = K / 2, srow = K / 32, arow = kActFP4 ? K / 2 : K;
  const int nss = (int)(K / 512);
  uint8_t* const stg = reinterpret_cast<uint8_t*>(&stg_all[wave][0]);
  // load instruction s gives lane 8 q + j row 8 (s & 1) + q and 16-byte block
  // 8 (s >> 1) + ((j + q) & 7) of the row's 256-byte super-step chunk; the lane's
  // MFMA operand of step s (row r16, block 4 s + g) is then read back at rd[s]
  const int q = lane >> 3, rot = ((lane & 7) + q) & 7;
  const uint32_t wvoff = (uint32_t)(q * wrow + 16 * rot);
  const uint32_t svoff = (uint32_t)(r16 * srow);
  int rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    rd[s] = (2 * (s >> 1) + (r16 >> 3)) * kStgStride + 128 * (r16 & 7) + 16 * ((4 * s + g - (r16 & 7)) & 7);

  int rank = 0;  // non-empty experts seen so far (wave-uniform)
  for (int c0 = 0; c0 < a.E; c0 += 256) {
    // lane l looks at experts c0 + 64 i + l, i = 0..3; mask i has bit b for expert c0 + 64 i + b
    int lo_l[4], cnt_l[4];
    unsigned long long mask[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = c0 + 64 * i + lane;
      lo_l[i] = 0;
      cnt_l[i] = 0;
      if (e < a.E) {
        lo_l[i] = a.offsets[e];
        cnt_l[i] = a.offsets[e + 1] - lo_l[i];
      }
      mask[i] = __ballot(cnt_l[i] > 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      unsigned long long m = mask[i];
      while (m) {
        const int b = __builtin_ctzll(m);
        m &= m - 1;
        if ((rank++ & 3) != wave) continue;
        const int e = c0 + 64 * i + b;
        const int lo = __builtin_amdgcn_readlane(lo_l[i], b);
        const int cnt = __builtin_amdgcn_readlane(cnt_l[i], b);
        // the expert's W2 rows n0 .. n0 + 15 (one expert's codes stay below 4 GiB: checked on the host)
        const int64_t rbase = (int64_t)e * a.H + n0;
        const buf_rsrc wr = make_rsrc(a.w2 + rbase * wrow, (uint32_t)(16 * wrow));
        const buf_rsrc sr = make_rsrc(a.w2_scale + rbase * srow, (uint32_t)(16 * srow));
        for (int m0 = 0; m0 < cnt; m0 += 16) {
          // h row lo + m0 + r16 (lanes past the expert's rows read row lo + m0; never stored)
          const int64_t hr = lo + m0 + (m0 + r16 < cnt ? r16 : 0);
          const uint8_t* ap = a.h + hr * arow + 16 * g;
          const uint8_t* asp = a.h_scale + hr * srow;
          v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
          for (int ss0 = 0; ss0 < nss; ss0 += CH) {
            // the weight loads of CH super-steps first, then the activations of the
            // first DA of them; the activations of super-step c + DA go out once step c
            // is done. A super-step past the end re-reads the last one and multiplies
            // it by zero activation codes.
            v4i raw[CH][4], sraw[CH], araw[CH][kAV], asraw[CH];
#pragma unroll
            for (int c = 0; c < CH; ++c) {
              const int ss = min(ss0 + c, nss - 1);
#pragma unroll
              for (int s = 0; s < 4; ++s)
                raw[c][s] = buf_load16_nt(wr, wvoff + 128 * (s >> 1), (uint32_t)(8 * (s & 1) * wrow + ss * 256));
              sraw[c] = buf_load16(sr, svoff, (uint32_t)(ss * 16));
            }
            auto load_act = [&](auto cc) {
              constexpr int c = decltype(cc)::value;
              const int ss = min(ss0 + c, nss - 1);
              if (kActFP4) {
#pragma unroll
                for (int s = 0; s < 4; ++s) araw[c][s] = *reinterpret_cast<const v4i*>(ap + (int64_t)ss * 256 + 64 * s);
              } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                  araw[c][2 * s] = *reinterpret_cast<const v4i*>(ap + (int64_t)ss * 512 + 128 * s);
                  araw[c][2 * s + 1] = *reinterpret_cast<const v4i*>(ap + (int64_t)ss * 512 + 128 * s + 64);
                }
              }
              asraw[c] = *reinterpret_cast<const v4i*>(asp + (int64_t)ss * 16);
            };
            static_for<0, DA>(load_act);
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, CH>([&](auto cc) {
              constexpr int c = decltype(cc)::value;
              const bool live = ss0 + c < nss;
#pragma unroll
              for (int s = 0; s < 4; ++s) *reinterpret_cast<v4i*>(stg + s * kStgStride + 16 * lane) = raw[c][s];
              v8i b[4];
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                const v4i x = *reinterpret_cast<const v4i*>(stg + rd[s]);
                b[s] = v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0};
              }
              const int as = fc2c_scales(asraw[c], g), bs = fc2c_scales(sraw[c], g);
              v8i av[4];
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                const v4i z = v4i{0, 0, 0, 0};
                const v4i lo4 = live ? araw[c][kActFP4 ? s : 2 * s] : z;
                const v4i hi4 = kActFP4 || !live ? z : araw[c][kActFP4 ? s : 2 * s + 1];
                av[s] = v8i{lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
              }
              acc = mfma16x16x128<kFA, kFmtFP4, 0>(av[0], b[0], acc, as, bs);
              acc = mfma16x16x128<kFA, kFmtFP4, 1>(av[1], b[1], acc, as, bs);
              acc = mfma16x16x128<kFA, kFmtFP4, 2>(av[2], b[2], acc, as, bs);
              acc = mfma16x16x128<kFA, kFmtFP4, 3>(av[3], b[3], acc, as, bs);
              if constexpr (c + DA < CH) load_act(std::integral_constant<int, c + DA>{});
            });
          }
          // acc[v] = y of the expert's row m0 + 4 g + v, column n0 + r16
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int row = m0 + 4 * g + v;
            if (row < cnt) ytab[a.sorted_pair[lo + row]][r16] = acc[v];
          }
        }
      }
    }
  }
  __syncthreads();
  // out[t][n0 + c] = sum_j gates[t][j] * y[t][j][c] over j = 0, 1, ... (fp32 fused multiply-adds)
  for (int idx = threadIdx.x; idx < a.T * 16; idx += 256) {
    const int t = idx >> 4, c = idx & 15;
    float s = 0.0f;
    for (int j = 0; j < a.topk; ++j) s = fmaf(a.gates[t * a.topk + j], ytab[t * a.topk + j][c], s);
    const int64_t o = (int64_t)t * a.H + n0 + c;
    if (a.out_bf16) static_cast<uint16_t*>(a.out)[o] = (uint16_t)bf16_round(s);
    else static_cast<float*>(a.out)[o] = s;
  }
}

int launch_fc2_combine(const uint8_t* h, const uint8_t* h_scale, bool act_fp4, int64_t T, int topk, int64_t H,
                       int64_t I, int E, const int32_t* offsets, const int32_t* sorted_pair, const float* gates,
                       const uint8_t* w2, const uint8_t* w2_scale, void* out, bool out_bf16, hipStream_t stream) {
  if (T <= 0) return 0;
  if (T * topk > fc2c::kMaxPairs || H % 16 != 0 || I % 512 != 0) return -1;
  const Fc2cArgs a{h, h_scale, w2, w2_scale, offsets, sorted_pair, gates, out, T, H, I, topk, E, out_bf16 ? 1 : 0};
  const dim3 grid((unsigned)(H / 16));
  if (act_fp4) fc2_combine_kernel<true, 4, 4><<<grid, 256, 0, stream>>>(a);
  else fc2_combine_kernel<false, 4, 2><<<grid, 256, 0, stream>>>(a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mxf

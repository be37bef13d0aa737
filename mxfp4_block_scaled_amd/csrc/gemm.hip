// Dispatch of the dense and grouped MXFP4 GEMMs: few rows per expert go to the
// weight-streaming kernel, many rows to the LDS-ring kernel.
#include "gemm_common.hpp"

namespace mxf {

// grouped GEMMs with few rows per expert: experts of at most this many rows (one 16-row
// fragment) go to the weight-streaming kernel
constexpr int kSplitRows = 16;

int dense_ksplit(int64_t M, int64_t N, int64_t K) {
  // M <= 64 streams the weights with 64 weight rows per workgroup: N / 64 workgroups
  // fill the chip only for very wide N, so K is also split into slices of 4
  // super-steps (one per wave), summed afterwards in a fixed order
  if (M <= 0 || M > 64 || N % 4 != 0) return 1;
  const int64_t nss = K / 512;
  return (int)(nss > 4 ? cdiv(nss, 4) : 1);
}

int dense_q_ksplit(int64_t M, int64_t N, int64_t K) {
  // a weight matrix of at most 1 MiB of codes is streamed by few workgroups over the
  // whole K in one launch (the slices' second launch would cost more than it saves)
  if (N * (K / 2) <= ((int64_t)1 << 20)) return 1;
  return dense_ksplit(M, N, K);
}

int launch_dense_q_gemm(const uint16_t* a16, bool act_fp4, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                        const uint8_t* w_scale, float* c, float* partials, hipStream_t stream) {
  if (M == 0) return 0;
  if (M > kDenseQRows) return -1;
  GemmArgs a{};
  a.act = reinterpret_cast<const uint8_t*>(a16);
  a.act_rows = M;
  a.M = M;
  a.w = w;
  a.w_scale = w_scale;
  a.K = K;
  a.N = N;
  a.E = 1;
  a.topk = 1;
  const int S = dense_q_ksplit(M, N, K);
  if (S > 1) {
    a.out = partials;
    a.kchunk = 4;
    launch_stream_q_gemm(act_fp4, a, dim3((unsigned)cdiv(N, 64), (unsigned)S), stream);
    launch_reduce_partials(partials, S, M * N, c, stream);
  } else {
    a.out = c;
    launch_stream_q_gemm(act_fp4, a, dim3((unsigned)cdiv(N, 64), 1), stream);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_dense_gemm(const uint8_t* qa, const uint8_t* qa_scale, bool act_fp4, int64_t M, int64_t N, int64_t K,
                      const uint8_t* w, const uint8_t* w_scale, float* c, float* partials, hipStream_t stream) {
  if (M == 0) return 0;
  GemmArgs a{};
  a.w = w;
  a.w_scale = w_scale;
  a.K = K;
  a.N = N;
  a.E = 1;
  a.topk = 1;
  const int64_t arow = act_fp4 ? K / 2 : K;
  if (M > 64 && N % tile::BN == 0) {
    a.act = qa;
    a.act_scale = qa_scale;
    a.out = c;
    a.M = M;
    a.act_rows = M;
    a.ntiles = (int)(N / tile::BN);
    if (launch_tile_gemm(kModeDense, false, act_fp4, a, M, 0, stream)) return -1;
  } else if (dense_ksplit(M, N, K) > 1) {
    const int S = dense_ksplit(M, N, K);
    a.act = qa;
    a.act_scale = qa_scale;
    a.out = partials;
    a.M = M;
    a.kchunk = 4;
    launch_stream_gemm(kModeDense, false, act_fp4, a, (int)cdiv(M, 16), dim3((unsigned)cdiv(N, 64), (unsigned)S), stream);
    launch_reduce_partials(partials, S, M * N, c, stream);
  } else {
    for (int64_t m0 = 0; m0 < M; m0 += 64) {
      const int64_t mm = M - m0 < 64 ? M - m0 : 64;
      a.act = qa + m0 * arow;
      a.act_scale = qa_scale + m0 * (K / 32);
      a.out = c + m0 * N;
      a.M = mm;
      launch_stream_gemm(kModeDense, false, act_fp4, a, (int)cdiv(mm, 16), dim3((unsigned)cdiv(N, 64), 1), stream);
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
  f1.act_rows = T;
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
  f2.act_rows = R;
  f2.act_scale = h_scale;
  f2.w = w2;
  f2.w_scale = w2_scale;
  f2.out = y;
  f2.K = I;
  f2.N = H;
  const int64_t slots = R < E ? R : E;
  if (T <= 64) {
    const int mt = (int)cdiv(T, 16);
    launch_stream_gemm(kModeFC1, false, act_fp4, f1, mt, dim3((unsigned)(I / 32), (unsigned)slots), stream);
    launch_stream_gemm(kModeFC2, y_bf16, act_fp4, f2, mt, dim3((unsigned)cdiv(H, 64), (unsigned)slots), stream);
  } else {
    // R rows over at most `slots` non-empty experts, each of which adds at most one partial unit
    f1.ntiles = (int)(I / (tile::BN / 2));
    f2.ntiles = (int)(H / tile::BN);
    // Fewer than 64 rows per expert on average (skewed routing): the experts of at most
    // 16 rows stream their weights through the one-fragment kernel at HBM rate instead
    // of each occupying a tile workgroup for a full weight tile; the tiled kernels take
    // the rest. Both pairs of launches size their grids for every expert and skip the
    // other class's.
    const bool split = R < 64 * (int64_t)E;
    if (split) {
      f1.split = f2.split = kSplitRows;
      launch_stream_gemm(kModeFC1, false, act_fp4, f1, 1, dim3((unsigned)(I / 32), (unsigned)slots), stream);
      launch_stream_gemm(kModeFC2, y_bf16, act_fp4, f2, 1, dim3((unsigned)cdiv(H, 64), (unsigned)slots), stream);
    }
    if (launch_tile_gemm(kModeFC1, false, act_fp4, f1, R, slots, stream)) return -1;
    if (launch_tile_gemm(kModeFC2, y_bf16, act_fp4, f2, R, slots, stream)) return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_grouped_gemm_combine(const uint8_t* q, const uint8_t* q_scale, bool act_fp4, int64_t T, int topk,
                                int64_t H, int64_t I, int E, const int32_t* expert_offsets,
                                const int32_t* sorted_pair, const int32_t* topk_ids, const int32_t* pair_row,
                                const float* gates, const uint8_t* w1,
                                const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale, uint8_t* h,
                                uint8_t* h_scale, void* out, bool out_bf16, hipStream_t stream) {
  if (T == 0) return 0;
  if (T > 64) return -1;
  GemmArgs f1{};
  f1.act = q;
  f1.act_rows = T;
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
  const int64_t R = T * topk, slots = R < E ? R : E;
  launch_stream_gemm(kModeFC1, false, act_fp4, f1, (int)cdiv(T, 16), dim3((unsigned)(I / 32), (unsigned)slots),
                     stream);
  return launch_fc2_combine(h, h_scale, act_fp4, T, topk, H, I, topk_ids, pair_row, gates, w2, w2_scale, out,
                            out_bf16, stream);
}

}  // namespace mxf

// extern "C" entry points: validate every argument, then enqueue the kernels.
// Nothing is enqueued when validation fails; the declarations and contracts
// are in include/mxfp4_moe.h.
#include "mxfp4_moe.h"

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(mxf_stream s) { return reinterpret_cast<hipStream_t>(s); }

inline bool valid_elem(int f) { return f == MXF_E4M3 || f == MXF_E2M1; }
inline bool valid_dtype(int d) { return d == MXF_F32 || d == MXF_BF16; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

}  // namespace

extern "C" {

const char* mxf_status_str(int status) {
  switch (status) {
    case MXF_OK: return "MXF_OK";
    case MXF_ERR_NULL: return "MXF_ERR_NULL: a required pointer is NULL";
    case MXF_ERR_SHAPE: return "MXF_ERR_SHAPE: a size is negative or not a multiple the kernels need";
    case MXF_ERR_ALIGN: return "MXF_ERR_ALIGN: a pointer is not 16-byte aligned";
    case MXF_ERR_FORMAT: return "MXF_ERR_FORMAT: unknown element format or dtype";
    case MXF_ERR_UNSUPPORTED: return "MXF_ERR_UNSUPPORTED: sizes outside what this library handles";
    case MXF_ERR_LAUNCH: return "MXF_ERR_LAUNCH: a kernel launch failed";
    case MXF_ERR_WORKSPACE: return "MXF_ERR_WORKSPACE: workspace missing or too small";
    default: return "unknown mxf_status";
  }
}

int mxf_abi_version(void) { return MXF_ABI_VERSION; }

int mxfp4_quantize_act(const void* x, int x_dtype, int64_t rows, int64_t K, int fmt, uint8_t* q,
                       uint8_t* q_scale, mxf_stream stream) {
  if (!valid_dtype(x_dtype) || !valid_elem(fmt)) return MXF_ERR_FORMAT;
  if (rows < 0 || K <= 0 || K % 32 != 0) return MXF_ERR_SHAPE;
  if (rows == 0) return MXF_OK;
  if (!x || !q || !q_scale) return MXF_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || !aligned16(q_scale)) return MXF_ERR_ALIGN;
  int rc = mxf::launch_quantize_act(x, x_dtype == MXF_F32, rows, K, fmt == MXF_E2M1, q, q_scale, as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}

size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_fmt) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if (M <= mxf::kDenseQRows) {  // quantised in registers: only the K-slice partials, if any
    const int S = mxf::dense_q_ksplit(M, N, K);
    return S > 1 ? round_up((size_t)S * (size_t)M * (size_t)N * sizeof(float), 256) : 0;
  }
  const size_t codes = (size_t)M * (size_t)(act_fmt == MXF_E2M1 ? K / 2 : K);
  const int S = mxf::dense_ksplit(M, N, K);
  const size_t partials = S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
  return round_up(codes, 256) + round_up((size_t)M * (size_t)(K / 32), 256) + round_up(partials, 256);
}

int mxfp4_gemm(const uint16_t* a, int64_t M, int64_t N, int64_t K, int act_fmt, const uint8_t* w,
               const uint8_t* w_scale, float* c, void* workspace, size_t workspace_bytes, mxf_stream stream) {
  if (!valid_elem(act_fmt)) return MXF_ERR_FORMAT;
  if (M < 0 || M > kMaxRows || N <= 0 || N % 16 != 0 || K <= 0 || K % 512 != 0) return MXF_ERR_SHAPE;
  if (M > 64 && N % 256 == 0 && !mxf::tile_offsets_fit(M, K, N, act_fmt == MXF_E2M1)) return MXF_ERR_UNSUPPORTED;
  // the streaming kernel addresses 64 weight rows of a workgroup with 32-bit offsets
  if ((M <= 64 || N % 256 != 0) && 64 * (K / 2) >= ((int64_t)1 << 32)) return MXF_ERR_UNSUPPORTED;
  if (M == 0) return MXF_OK;
  if (!a || !w || !w_scale || !c) return MXF_ERR_NULL;
  if (!aligned16(a) || !aligned16(w) || !aligned16(w_scale) || !aligned16(c)) return MXF_ERR_ALIGN;
  const size_t need = mxfp4_gemm_workspace_bytes(M, N, K, act_fmt);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return MXF_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MXF_ERR_ALIGN;
  }
  const bool fp4 = act_fmt == MXF_E2M1;
  hipStream_t s = as_stream(stream);
  if (M <= mxf::kDenseQRows) {
    return mxf::launch_dense_q_gemm(a, fp4, M, N, K, w, w_scale, c, static_cast<float*>(workspace), s)
               ? MXF_ERR_LAUNCH
               : MXF_OK;
  }
  uint8_t* qa = static_cast<uint8_t*>(workspace);
  uint8_t* qs = qa + round_up((size_t)M * (size_t)(act_fmt == MXF_E2M1 ? K / 2 : K), 256);
  float* part = reinterpret_cast<float*>(qs + round_up((size_t)M * (size_t)(K / 32), 256));
  if (mxf::launch_quantize_act(a, false, M, K, fp4, qa, qs, s)) return MXF_ERR_LAUNCH;
  if (mxf::launch_dense_gemm(qa, qs, fp4, M, N, K, w, w_scale, c, part, s)) return MXF_ERR_LAUNCH;
  return MXF_OK;
}

size_t fp4_w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const int S = mxf::w4a16_ksplit(M, N, K);
  const int64_t mm = M < 64 ? M : 64;
  return S > 1 ? round_up((size_t)S * (size_t)mm * (size_t)N * sizeof(float), 256) : 0;
}

namespace {
int w4a16_call(bool nvfp4, const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w,
               const uint8_t* w_scale, float* c, void* workspace, size_t workspace_bytes, mxf_stream stream) {
  if (M < 0 || M > kMaxRows || N <= 0 || N % 16 != 0 || K <= 0 || K % 512 != 0) return MXF_ERR_SHAPE;
  // 64 weight rows of a workgroup are addressed with 32-bit offsets
  if (64 * (K / 2) >= ((int64_t)1 << 32)) return MXF_ERR_UNSUPPORTED;
  if (M == 0) return MXF_OK;
  if (!a || !w || !w_scale || !c) return MXF_ERR_NULL;
  if (!aligned16(a) || !aligned16(w) || !aligned16(w_scale) || !aligned16(c)) return MXF_ERR_ALIGN;
  const size_t need = fp4_w4a16_workspace_bytes(M, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MXF_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return MXF_ERR_ALIGN;
  const int rc = mxf::launch_w4a16_gemm(nvfp4, a, M, N, K, w, w_scale, c, static_cast<float*>(workspace),
                                        as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}
}  // namespace

int mxfp4_gemm_w4a16(const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w, const uint8_t* w_scale,
                     float* c, void* workspace, size_t workspace_bytes, mxf_stream stream) {
  return w4a16_call(false, a, M, N, K, w, w_scale, c, workspace, workspace_bytes, stream);
}

int nvfp4_gemm_w4a16(const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w, const uint8_t* w_scale,
                     float* c, void* workspace, size_t workspace_bytes, mxf_stream stream) {
  return w4a16_call(true, a, M, N, K, w, w_scale, c, workspace, workspace_bytes, stream);
}

int q8_quantize_act(const uint16_t* x, int64_t rows, int64_t K, int8_t* q, uint16_t* d, mxf_stream stream) {
  if (rows < 0 || K <= 0 || K % 32 != 0) return MXF_ERR_SHAPE;
  if (rows == 0) return MXF_OK;
  if (!x || !q || !d) return MXF_ERR_NULL;
  if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(d) & 1u)) return MXF_ERR_ALIGN;
  return mxf::launch_q8_quantize(x, rows, K, q, d, as_stream(stream)) ? MXF_ERR_LAUNCH : MXF_OK;
}

size_t mxfp4_gemm_q8_workspace_bytes(int64_t M, int64_t N, int64_t K) { return fp4_w4a16_workspace_bytes(M, N, K); }

int mxfp4_gemm_q8(const int8_t* q, const uint16_t* d, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                  const uint8_t* w_scale, float* c, void* workspace, size_t workspace_bytes, mxf_stream stream) {
  if (M < 0 || M > kMaxRows || N <= 0 || N % 16 != 0 || K <= 0 || K % 512 != 0) return MXF_ERR_SHAPE;
  if (64 * (K / 2) >= ((int64_t)1 << 32)) return MXF_ERR_UNSUPPORTED;
  if (M == 0) return MXF_OK;
  if (!q || !d || !w || !w_scale || !c) return MXF_ERR_NULL;
  if (!aligned16(q) || !aligned16(d) || !aligned16(w) || !aligned16(w_scale) || !aligned16(c)) return MXF_ERR_ALIGN;
  const size_t need = mxfp4_gemm_q8_workspace_bytes(M, N, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MXF_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return MXF_ERR_ALIGN;
  const int rc = mxf::launch_q8_gemm(q, d, M, N, K, w, w_scale, c, static_cast<float*>(workspace), as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}

int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t topk, int32_t* topk_ids, float* gates,
                      int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row, mxf_stream stream) {
  if (T < 0 || E < 1 || topk < 1 || topk > 8 || topk > E) return MXF_ERR_SHAPE;
  if (E > 1024 || T * (int64_t)topk > kMaxRows) return MXF_ERR_UNSUPPORTED;
  if (!expert_offsets) return MXF_ERR_NULL;
  if (T > 0 && (!logits || !topk_ids || !gates || !sorted_pair || !pair_row)) return MXF_ERR_NULL;
  if (!aligned16(expert_offsets)) return MXF_ERR_ALIGN;
  if (T > 0 && (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(gates) || !aligned16(sorted_pair) ||
                !aligned16(pair_row)))
    return MXF_ERR_ALIGN;
  if (!mxf::route_permute_supported(T, E, topk)) return MXF_ERR_UNSUPPORTED;
  int rc = mxf::launch_route_permute(logits, T, E, topk, topk_ids, gates, expert_offsets, sorted_pair, pair_row,
                                     as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}

int moe_quantize_route(const void* x, int x_dtype, const float* logits, int64_t T, int64_t H, int32_t E,
                       int32_t topk, int act_fmt, uint8_t* q, uint8_t* q_scale, int32_t* topk_ids, float* gates,
                       int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_row, mxf_stream stream) {
  if (!valid_dtype(x_dtype) || !valid_elem(act_fmt)) return MXF_ERR_FORMAT;
  if (T < 0 || H <= 0 || H % 32 != 0 || E < 1 || topk < 1 || topk > 8 || topk > E) return MXF_ERR_SHAPE;
  if (!mxf::quantize_route_supported(T, E)) return MXF_ERR_UNSUPPORTED;
  if (!expert_offsets) return MXF_ERR_NULL;
  if (T > 0 && (!x || !logits || !q || !q_scale || !topk_ids || !gates || !sorted_pair || !pair_row))
    return MXF_ERR_NULL;
  if (!aligned16(expert_offsets)) return MXF_ERR_ALIGN;
  if (T > 0) {
    const void* ptrs[] = {x, logits, q, q_scale, topk_ids, gates, sorted_pair, pair_row};
    for (const void* p : ptrs)
      if (!aligned16(p)) return MXF_ERR_ALIGN;
  }
  int rc = mxf::launch_quantize_route(x, x_dtype == MXF_F32, H, act_fmt == MXF_E2M1, q, q_scale, logits, T, E, topk,
                                      topk_ids, gates, expert_offsets, sorted_pair, pair_row, as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}

int moe_grouped_mxfp4_gemm(const uint8_t* q, const uint8_t* q_scale, int act_fmt, int64_t T, int32_t topk,
                           int64_t H, int64_t I, int32_t E, const int32_t* expert_offsets,
                           const int32_t* sorted_pair, const uint8_t* w1, const uint8_t* w1_scale,
                           const uint8_t* w2, const uint8_t* w2_scale, uint8_t* h, uint8_t* h_scale, void* y,
                           int y_dtype, mxf_stream stream) {
  if (!valid_elem(act_fmt) || !valid_dtype(y_dtype)) return MXF_ERR_FORMAT;
  if (T < 0 || topk < 1 || topk > 8 || E < 1 || topk > E) return MXF_ERR_SHAPE;
  if (H <= 0 || H % 512 != 0 || I <= 0 || I % 512 != 0) return MXF_ERR_SHAPE;
  if (E > 1024 || T * (int64_t)topk > kMaxRows) return MXF_ERR_UNSUPPORTED;
  // one expert's w1 and w2 codes are addressed with 32-bit offsets by every kernel
  if (2 * I * (H / 2) >= ((int64_t)1 << 32) || H * (I / 2) >= ((int64_t)1 << 32)) return MXF_ERR_UNSUPPORTED;
  if (T > 64 && (!mxf::tile_offsets_fit(T, H, 2 * I, act_fmt == MXF_E2M1) ||
                 !mxf::tile_offsets_fit(T * topk, I, H, act_fmt == MXF_E2M1)))
    return MXF_ERR_UNSUPPORTED;
  if (T == 0) return MXF_OK;
  if (!q || !q_scale || !expert_offsets || !sorted_pair || !w1 || !w1_scale || !w2 || !w2_scale || !h ||
      !h_scale || !y)
    return MXF_ERR_NULL;
  const void* ptrs[] = {q, q_scale, expert_offsets, sorted_pair, w1, w1_scale, w2, w2_scale, h, h_scale, y};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MXF_ERR_ALIGN;
  int rc = mxf::launch_grouped_gemm(q, q_scale, act_fmt == MXF_E2M1, T, topk, H, I, E, expert_offsets, sorted_pair,
                                    w1, w1_scale, w2, w2_scale, h, h_scale, y, y_dtype == MXF_BF16,
                                    as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}

int moe_grouped_mxfp4_gemm_combine(const uint8_t* q, const uint8_t* q_scale, int act_fmt, int64_t T, int32_t topk,
                                   int64_t H, int64_t I, int32_t E, const int32_t* expert_offsets,
                                   const int32_t* sorted_pair, const int32_t* topk_ids, const int32_t* pair_row,
                                   const float* gates, const uint8_t* w1,
                                   const uint8_t* w1_scale, const uint8_t* w2, const uint8_t* w2_scale, uint8_t* h,
                                   uint8_t* h_scale, void* out, int out_dtype, mxf_stream stream) {
  if (!valid_elem(act_fmt) || !valid_dtype(out_dtype)) return MXF_ERR_FORMAT;
  if (T < 0 || topk < 1 || topk > 8 || E < 1 || topk > E) return MXF_ERR_SHAPE;
  if (H <= 0 || H % 512 != 0 || I <= 0 || I % 512 != 0) return MXF_ERR_SHAPE;
  if (E > 1024 || T > 64) return MXF_ERR_UNSUPPORTED;
  if (2 * I * (H / 2) >= ((int64_t)1 << 32) || H * (I / 2) >= ((int64_t)1 << 32)) return MXF_ERR_UNSUPPORTED;
  if (T == 0) return MXF_OK;
  if (!q || !q_scale || !expert_offsets || !sorted_pair || !topk_ids || !pair_row || !gates || !w1 || !w1_scale ||
      !w2 || !w2_scale || !h || !h_scale || !out)
    return MXF_ERR_NULL;
  const void* ptrs[] = {q,  q_scale,  expert_offsets, sorted_pair, topk_ids, pair_row, gates,
                        w1, w1_scale, w2,             w2_scale,    h,        h_scale,  out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MXF_ERR_ALIGN;
  int rc = mxf::launch_grouped_gemm_combine(q, q_scale, act_fmt == MXF_E2M1, T, topk, H, I, E, expert_offsets,
                                            sorted_pair, topk_ids, pair_row, gates, w1, w1_scale, w2, w2_scale, h,
                                            h_scale, out,
                                            out_dtype == MXF_BF16, as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}

int moe_unpermute_combine(const void* y, int y_dtype, const float* gates, const int32_t* pair_row, int64_t T,
                          int32_t topk, int64_t H, void* out, int out_dtype, mxf_stream stream) {
  if (!valid_dtype(y_dtype) || !valid_dtype(out_dtype)) return MXF_ERR_FORMAT;
  if (T < 0 || topk < 1 || topk > 8 || H <= 0 || H % 8 != 0) return MXF_ERR_SHAPE;
  if (T * (int64_t)topk > kMaxRows) return MXF_ERR_UNSUPPORTED;
  if (T == 0) return MXF_OK;
  if (!y || !gates || !pair_row || !out) return MXF_ERR_NULL;
  if (!aligned16(y) || !aligned16(gates) || !aligned16(pair_row) || !aligned16(out)) return MXF_ERR_ALIGN;
  int rc = mxf::launch_combine(y, y_dtype == MXF_BF16, gates, pair_row, T, topk, H, out, out_dtype == MXF_BF16,
                               as_stream(stream));
  return rc ? MXF_ERR_LAUNCH : MXF_OK;
}

}  // extern "C"

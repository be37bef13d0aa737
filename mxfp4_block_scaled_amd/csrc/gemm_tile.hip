// Dispatch of the tiled GEMMs (many rows per weight matrix: grouped prefill, dense
// M > 64): E2M1 activations go to the 256 x 256 ring kernel of 256-k stages
// (gemm_wide.hip), E4M3 activations to the 256 x 256 ring kernel of 128-k stages
// (gemm_f8ring.hip).
#include "gemm_common.hpp"

namespace mxf {

// Both kernels address the activation matrix and one expert's weight matrix with
// 32-bit byte offsets (raw buffer resources): callers check tile_offsets_fit first.
// Measured on the 2048-token Zipf layer against the earlier 128 x 256 kernel whose
// weights went from HBM straight into registers: tiled FC1 509 -> 486 us, FC2
// 317 -> 282 us.
bool tile_offsets_fit(int64_t rows, int64_t K, int64_t N, bool act_fp4) {
  const int64_t lim = (int64_t)1 << 32;
  return rows * (act_fp4 ? K / 2 : K) < lim && N * (K / 2) < lim;
}

int launch_tile_gemm(int mode, bool y_bf16, bool act_fp4, const GemmArgs& a, int64_t rows, int64_t groups,
                     hipStream_t stream) {
  if (!tile_offsets_fit(a.act_rows, a.K, a.N, act_fp4)) return -1;
  if (act_fp4) {
    // 256-row units: an upper bound on the units summed over the groups
    launch_wide_gemm(mode, y_bf16, a, cdiv(rows, 256) + groups, stream);
    return 0;
  }
  // E4M3 activations: the 256 x 256 ring kernel of 128-k stages (gemm_f8ring.hip)
  launch_f8ring_gemm(mode, y_bf16, a, cdiv(rows, 256) + groups, stream);
  return 0;
}

}  // namespace mxf

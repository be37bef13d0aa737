/*
 * mxfp4_moe.h - C ABI of the MI355X (gfx950) MXFP4 mixture-of-experts expert path.
 *
 * The library computes the hot path of a DeepSeek-V4-Flash-style MoE layer whose
 * routed-expert weights are MXFP4: E2M1 codes (1 sign / 2 exponent / 1 mantissa
 * bit) with one UE8M0 scale per 32 K-elements, fed to block-scaled matrix
 * instructions without dequantisation to a 16-bit type
 * (page "DGX Spark 原生 FP4 矩阵指令：DwarfStar 如何利用 Blackwell 加速推理",
 * sections 一 and 二). Each token goes to the top-6 of 256 experts and runs two
 * FC contractions per expert (page "【DeepSeek V4】Triton FP4 优化实战：近距离感受
 * 老黄的刀法", "FP4 MoE GEMM 是什么？"); SwiGLU and the FP8 requantisation are
 * fused between them (page "Domestic GPUs are awesome! Moore thread full-link
 * adaptation DeepSeek-V4": "SwiGLU + FP8 quant", routing, dispatch/combine).
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers to caller-owned, contiguous, row-major buffers.
 *    The library never allocates, frees, copies to the host or synchronises.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the legacy
 *    default stream). Nothing is read back to the host: counts and offsets stay
 *    on the device.
 *  - Every argument is validated before anything is enqueued. On any error the
 *    function returns a non-zero mxf_status and enqueues nothing (no silent
 *    fallback to another path - the pages' FP4 path errors out on a K it cannot
 *    take, page "DGX Spark 原生 FP4 矩阵指令" section 三). MXF_ERR_LAUNCH means a
 *    launch failed after validation; device faults surface at the caller's next
 *    synchronisation.
 *  - Byte layouts:
 *      E4M3 activations   [rows][K]     u8, one OCP E4M3FN code per element
 *      E2M1 activations   [rows][K/2]   u8, element 2n in the low nibble of byte n
 *                                           (page "【DeepSeek V4】Triton FP4 优化实战",
 *                                           "第二步": even column = low nibble)
 *      UE8M0 scales       [rows][K/32]  u8, value 2^(byte - 127)
 *      MXFP4 weights      [N][K/2] codes + [N][K/32] scales, K contiguous ("nt")
 *  - Quantisation rule (OCP MX): per 32-element block, scale byte =
 *    clamp(floor(log2 amax) - emax + 127, 0, 254) (0 when amax = 0; emax = 8 for
 *    E4M3, 2 for E2M1), elements rounded to nearest even on the element grid,
 *    saturating at the largest normal (448 / 6), sign kept.
 *  - Alignment: every code and scale pointer must be 16-byte aligned, every
 *    fp32/bf16 pointer 16-byte aligned (128-bit loads and stores).
 */
#ifndef MXFP4_MOE_H
#define MXFP4_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXF_OK = 0,
  MXF_ERR_NULL = 1,        /* a required pointer is NULL */
  MXF_ERR_SHAPE = 2,       /* a size is negative, or not a multiple the kernels need */
  MXF_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  MXF_ERR_FORMAT = 4,      /* unknown element format or dtype enum */
  MXF_ERR_UNSUPPORTED = 5, /* valid arguments outside the sizes this library handles */
  MXF_ERR_LAUNCH = 6,      /* a kernel launch failed (hipGetLastError) */
  MXF_ERR_WORKSPACE = 7    /* workspace missing or smaller than required */
} mxf_status;

typedef enum { MXF_E4M3 = 0, MXF_E2M1 = 1 } mxf_elem;   /* activation element format */
typedef enum { MXF_F32 = 0, MXF_BF16 = 1 } mxf_dtype;   /* floating-point buffer type */

typedef void* mxf_stream; /* a hipStream_t */

/* Human-readable name of a status code (static storage, never NULL). */
const char* mxf_status_str(int status);

/* ABI version of this header (bumped on any signature change). */
int mxf_abi_version(void);
#define MXF_ABI_VERSION 2

/*
 * mxfp4_quantize_act - quantise activation rows per 32-element block.
 *   x        [rows][K] bf16 (x_dtype = MXF_BF16) or fp32 (MXF_F32) values
 *   fmt      MXF_E4M3 -> q [rows][K] ; MXF_E2M1 -> q [rows][K/2] (packed)
 *   q_scale  [rows][K/32] UE8M0 bytes
 * Bit-exact with the OCP MX rule above. Requires K % 32 == 0; rows == 0 is a
 * no-op. Errors: NULL, SHAPE (K % 32, negative sizes), FORMAT, ALIGN.
 */
int mxfp4_quantize_act(const void* x, int x_dtype, int64_t rows, int64_t K, int fmt,
                       uint8_t* q, uint8_t* q_scale, mxf_stream stream);

/*
 * mxfp4_gemm - dense MXFP4 GEMM, C = A_hat * W_hat^T
 * (the dense MXFP4 entry of page "DGX Spark 原生 FP4 矩阵指令" section 二).
 *   a        [M][K] bf16 activations, quantised inside the call per 32-block to
 *            act_fmt (E4M3 or E2M1) with the rule above; the quantised copy
 *            lives only in `workspace`
 *   w        [N][K/2] E2M1 codes, w_scale [N][K/32] UE8M0
 *   c        [M][N] fp32 output (fp32 accumulation of exact products)
 *   workspace, workspace_bytes: device scratch of at least
 *            mxfp4_gemm_workspace_bytes(M, N, K, act_fmt) bytes (16-byte
 *            aligned): the quantised activations and, for M <= 64, the fp32
 *            partial sums of the K slices; its contents on entry are ignored and
 *            on exit undefined. The slice sums are added in a fixed order, so
 *            results are bit-identical from run to run.
 * Requires K % 512 == 0 (one 512-k super-step of scaled-MFMA K steps) and
 * N % 16 == 0; M >= 0 (M == 0 is a no-op). For M > 64 with N % 256 == 0 (the
 * tiled kernels) the quantised activations and the weight codes must each stay
 * below 4 GiB, else UNSUPPORTED; otherwise (the weight-streaming kernel) 64
 * weight rows must stay below 4 GiB (K < 2^27), else UNSUPPORTED.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, WORKSPACE, UNSUPPORTED.
 */
size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int act_fmt);
int mxfp4_gemm(const uint16_t* a, int64_t M, int64_t N, int64_t K, int act_fmt,
               const uint8_t* w, const uint8_t* w_scale, float* c,
               void* workspace, size_t workspace_bytes, mxf_stream stream);

/*
 * moe_route_permute - top-k routing and the expert-grouped permutation.
 *   logits         [T][E] fp32
 *   topk_ids       [T][topk] i32: per token the topk largest logits, distinct
 *                  experts, ordered by (logit descending, expert index ascending)
 *   gates          [T][topk] fp32: softmax over the selected logits
 *                  (exp(l_j - l_0) / sum_j' exp(l_j' - l_0))
 *   expert_offsets [E+1] i32: exclusive prefix sum of per-expert pair counts
 *   sorted_pair    [T*topk] i32: pairs p = t*topk + j grouped by expert,
 *                  ascending p inside an expert (stable)
 *   pair_row       [T*topk] i32: inverse of sorted_pair
 * The integer outputs are bit-exact (deterministic). sorted_pair is also used
 * as scratch while the call runs. Requires 1 <= topk <= min(E, 8), E <= 1024,
 * T*topk < 2^31; T == 0 writes only expert_offsets (all zero). Errors: NULL,
 * SHAPE, ALIGN, UNSUPPORTED.
 */
int moe_route_permute(const float* logits, int64_t T, int32_t E, int32_t topk,
                      int32_t* topk_ids, float* gates, int32_t* expert_offsets,
                      int32_t* sorted_pair, int32_t* pair_row, mxf_stream stream);

/*
 * moe_grouped_mxfp4_gemm - both expert FCs for every (token, expert) pair.
 *   q, q_scale     quantised layer input [T][H] (E4M3) or [T][H/2] (E2M1) + [T][H/32]
 *   act_fmt        element format of q and of h
 *   expert_offsets, sorted_pair  as written by moe_route_permute
 *   w1, w1_scale   [E][2I][H/2], [E][2I][H/32]: rows 0..I-1 gate, I..2I-1 up
 *   w2, w2_scale   [E][H][I/2],  [E][H][I/32]
 *   h, h_scale     output workspace [T*topk][I] (E4M3) or [T*topk][I/2] (E2M1)
 *                  + [T*topk][I/32]: silu(gate) * up requantised per 32 along I
 *   y              [T*topk][H] fp32 or bf16 (y_dtype): FC2 output in the
 *                  permuted (expert-grouped) row order
 * Row r of the permuted order is token sorted_pair[r] / topk. The grid is sized
 * from T and topk; per-expert counts are read on the device.
 * Requires H % 512 == 0, I % 512 == 0, 1 <= topk <= min(E, 8), E <= 1024;
 * one expert's w1 and w2 codes must each stay below 4 GiB, and for T > 64 (the
 * tiled kernels) so must q and h, else UNSUPPORTED. T == 0 is a no-op.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, UNSUPPORTED.
 */
int moe_grouped_mxfp4_gemm(const uint8_t* q, const uint8_t* q_scale, int act_fmt,
                           int64_t T, int32_t topk, int64_t H, int64_t I, int32_t E,
                           const int32_t* expert_offsets, const int32_t* sorted_pair,
                           const uint8_t* w1, const uint8_t* w1_scale,
                           const uint8_t* w2, const uint8_t* w2_scale,
                           uint8_t* h, uint8_t* h_scale,
                           void* y, int y_dtype, mxf_stream stream);

/*
 * moe_unpermute_combine - out[t] = sum_{j=0..topk-1} gates[t][j] * y[pair_row[t*topk+j]]
 * accumulated in fp32 in slot order j = 0, 1, ..., then stored as out_dtype
 * (bf16: round to nearest even). y [T*topk][H] (y_dtype), out [T][H].
 * Requires H % 8 == 0. Errors: NULL, SHAPE, ALIGN, FORMAT.
 */
int moe_unpermute_combine(const void* y, int y_dtype, const float* gates,
                          const int32_t* pair_row, int64_t T, int32_t topk, int64_t H,
                          void* out, int out_dtype, mxf_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_MOE_H */

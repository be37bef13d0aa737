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
 * Defined by: the activation side of the FP4 path, page "DGX Spark 原生 FP4 矩阵
 * 指令" sections 一 (E2M1 elements with one UE8M0 scale per block, fed to the
 * matrix instruction as they are) and 二 (activations kept in FP4 end to end on the
 * FP4 path); the FP8 activations of the grouped FP8 x FP4 GEMM, page "【DeepSeek
 * V4】Triton FP4 优化实战" section 第零步 (the profiled m_grouped_fp8_fp4 call); and
 * the "FP8 quant" step of page "Domestic GPUs are awesome! ... DeepSeek-V4". The
 * block rule itself (floor(log2 amax) - emax, round to nearest even) is the OCP MX
 * one stated at the top of this header.
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
 * Defined by: the dense MXFP4 entry of page "DGX Spark 原生 FP4 矩阵指令" section 二,
 * the K-shape guard of its section 三 (a K the kernels cannot take is an error, never
 * a silent other path), and the dense shapes of the accuracy table in page "【DeepSeek
 * V4】Triton FP4 优化实战" section 第二步 (16 x 32 x 4096 and 64 x 4096 x 7168).
 *   a        [M][K] bf16 activations, quantised inside the call per 32-block to
 *            act_fmt (E4M3 or E2M1) with the rule above. For M <= 16 the GEMM
 *            kernel quantises them in registers and the codes are never written;
 *            for larger M the quantised copy lives only in `workspace`
 *   w        [N][K/2] E2M1 codes, w_scale [N][K/32] UE8M0
 *   c        [M][N] fp32 output (fp32 accumulation of exact products)
 *   workspace, workspace_bytes: device scratch of at least
 *            mxfp4_gemm_workspace_bytes(M, N, K, act_fmt) bytes (16-byte
 *            aligned; may be NULL when that is 0): the quantised activations
 *            (M > 16) and the fp32 partial sums of the K slices (M <= 64 with a
 *            long K; for M <= 16 only when the weight codes exceed 1 MiB - below
 *            that the call is one launch and needs no workspace); its contents on
 *            entry are ignored and on exit undefined. The slice sums are added in
 *            a fixed order, so results are bit-identical from run to run.
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
 * mxfp4_gemm_noalloc - mxfp4_gemm with its workspace inside the library.
 * For callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation. The
 * result is that of mxfp4_gemm (the same kernels, bit for bit).
 *   The workspace is a fixed device array of MXF_NOALLOC_SCRATCH_BYTES (16 MiB) per
 *   GPU, held from the library's first use on that GPU until the process ends; its
 *   device address is looked up once per device on the first call made with that
 *   device current. Nothing is allocated or freed by any call.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time on one
 *   GPU (different streams, or different host threads) race and give undefined
 *   results; calls ordered on one stream are safe. Nothing in the array needs to
 *   start at zero (each call overwrites what it reads).
 * Arguments as for mxfp4_gemm without the workspace pair. A call whose workspace
 * (mxfp4_gemm_workspace_bytes) exceeds the array returns MXF_ERR_WORKSPACE before
 * touching the device (the 64 x 4096 x 7168 GEMM needs 4.5 MiB). Other errors as
 * for mxfp4_gemm; MXF_ERR_LAUNCH also if the array's address cannot be found.
 */
#define MXF_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
size_t mxfp4_noalloc_scratch_bytes(void);
int mxfp4_gemm_noalloc(const uint16_t* a, int64_t M, int64_t N, int64_t K, int act_fmt,
                       const uint8_t* w, const uint8_t* w_scale, float* c, mxf_stream stream);

/*
 * mxfp4_gemm_w4a16 / nvfp4_gemm_w4a16 - FP4 weights x bf16 activations:
 *   C[M][N] (fp32) = A . W_hat^T, A [M][K] bf16 used as given (no activation
 *   quantisation), fp32 accumulation.
 * Defined by: the fused dequantise + matmul of page "【DeepSeek V4】Triton FP4 优化实战"
 * section 第二步 (packed FP4 weights, even column in the low nibble, turned into bf16
 * inside the kernel and multiplied in bf16, no 16-bit weight copy in memory), with its
 * accuracy table's shapes (1 x 32 x 4096, 1 x 4096 x 7168, 64 x 4096 x 7168); the
 * NVFP4 block format is the one of the kind::mxf4nvf4 / scale_vec::4X instruction of page
 * "DGX Spark 原生 FP4 矩阵指令" section 一 (E2M1 codes, a UE4M3 scale per 16 elements).
 *   w        [N][K/2] E2M1 codes, element 2n in the low nibble of byte n
 *   w_scale  mxfp4: [N][K/32] UE8M0 bytes, value 2^(byte - 127), bytes 2 .. 252 (every
 *            decoded weight then lies in bf16's normal range; smaller bytes give weights
 *            the bf16 instruction may flush, larger ones overflow bf16);
 *            nvfp4: [N][K/16] UE4M3 bytes (OCP E4M3 with the sign bit clear), value
 *            2^(e-7) (1 + m/8), or m 2^-9 for e = 0; 0x7F (NaN) is not a valid scale
 *   c        [M][N] fp32
 *   workspace, workspace_bytes: device scratch of at least fp4_w4a16_workspace_bytes(M,
 *            N, K) bytes (0 means none needed; 16-byte aligned): fp32 partial sums of
 *            the K slices, added in a fixed order (bit-identical results run to run).
 * Every weight value code x scale is exact in bf16, so the only rounding is the fp32
 * accumulation. Requires K % 512 == 0, N % 16 == 0, M >= 0 (0 is a no-op), K < 2^27.
 * Errors: NULL, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED.
 */
size_t fp4_w4a16_workspace_bytes(int64_t M, int64_t N, int64_t K);
int mxfp4_gemm_w4a16(const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                     const uint8_t* w_scale, float* c, void* workspace, size_t workspace_bytes,
                     mxf_stream stream);
int nvfp4_gemm_w4a16(const uint16_t* a, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                     const uint8_t* w_scale, float* c, void* workspace, size_t workspace_bytes,
                     mxf_stream stream);

/*
 * q8_quantize_act / mxfp4_gemm_q8 - the lookup-table route: Q8 activations x MXFP4
 * weights through int8 products.
 * Defined by: the generic FP4 path of hardware without FP4 matrix instructions, page
 * "DGX Spark 原生 FP4 矩阵指令" sections 二 and 三 (FP4 weights expanded to Q8-style
 * integers, Q8_1-style activations, lossless and with no FP4 speed bonus); the Q8_0
 * block (32 int8 + an fp16 scale) and the exact FP4 <-> 4-bit lookup-table equivalence,
 * page "企业官网建设流程全解析" sections 四 and 五.
 * q8_quantize_act:
 *   x  [rows][K] bf16; q [rows][K] int8; d [rows][K/32] fp16 (2-byte aligned)
 *   per 32-block: d = fp16(amax / 127) (fp32 quotient, round to nearest even),
 *   q = clamp(round_to_nearest_even(x / d), -127, 127) with the quotient in fp32, and
 *   q = 0 where d = 0. Bit-exact. Requires K % 32 == 0. Errors: NULL, SHAPE, ALIGN.
 *   (Q8_1's second per-block number, d times the sum of q, serves asymmetric weight
 *   formats; E2M1 is symmetric, so it is not formed.)
 * mxfp4_gemm_q8:
 *   C[M][N] (fp32) = sum over 32-blocks b of (sum_k q[m][k] w8[n][k]) d[m][b] 2^(e - 128)
 *   where w8 = 2 x e2m1(code) in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12} (a 16-entry table)
 *   and e the weight's UE8M0 byte (bytes 2 .. 252): w8 2^(e - 128) is the MXFP4 weight
 *   exactly. Each block's integer sum is exact; the scaling and the sum over blocks
 *   round in fp32. q, d as written by q8_quantize_act (d 16-byte aligned here); w, w_scale
 *   as for mxfp4_gemm; workspace >= mxfp4_gemm_q8_workspace_bytes(M, N, K) (K-slice
 *   partial sums, added in a fixed order). Requires K % 512 == 0, N % 16 == 0,
 *   K < 2^27. Errors: NULL, SHAPE, ALIGN, WORKSPACE, UNSUPPORTED.
 */
int q8_quantize_act(const uint16_t* x, int64_t rows, int64_t K, int8_t* q, uint16_t* d, mxf_stream stream);
size_t mxfp4_gemm_q8_workspace_bytes(int64_t M, int64_t N, int64_t K);
int mxfp4_gemm_q8(const int8_t* q, const uint16_t* d, int64_t M, int64_t N, int64_t K, const uint8_t* w,
                  const uint8_t* w_scale, float* c, void* workspace, size_t workspace_bytes, mxf_stream stream);

/*
 * moe_route_permute - top-k routing and the expert-grouped permutation.
 * Defined by: page "【DeepSeek V4】Triton FP4 优化实战" section "FP4 MoE GEMM 是什么？"
 * (each token picks 6 of 256 experts) and page "Domestic GPUs are awesome! ...
 * DeepSeek-V4" (MoE routing / Top-k as an operator, and the dispatch that groups a
 * token's rows by expert before the expert GEMMs); the grouped, row-contiguous
 * layout is the one of the profiled m_grouped_..._contiguous call in the Triton
 * page's section 第零步.
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
 * moe_quantize_route - mxfp4_quantize_act of the layer input and moe_route_permute
 * of its router logits in one launch, for decode-sized batches.
 * Defined by: the two calls above (the same steps, outputs bit-identical to them);
 * the two steps share no data, so one launch replaces two (at decode sizes a
 * launch's fixed cost is most of either step's time).
 *   x [T][H] bf16 or fp32 (x_dtype); logits [T][E] fp32
 *   q, q_scale     [T][H] (E4M3) or [T][H/2] (E2M1), [T][H/32], as mxfp4_quantize_act
 *   topk_ids, gates, expert_offsets, sorted_pair, pair_row   as moe_route_permute
 * Requires T <= 64 and E <= 256 (else UNSUPPORTED: use the two calls), H % 32 == 0,
 * 1 <= topk <= min(E, 8). expert_offsets is written (all zero) even when T == 0.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, UNSUPPORTED.
 */
int moe_quantize_route(const void* x, int x_dtype, const float* logits, int64_t T, int64_t H,
                       int32_t E, int32_t topk, int act_fmt, uint8_t* q, uint8_t* q_scale,
                       int32_t* topk_ids, float* gates, int32_t* expert_offsets,
                       int32_t* sorted_pair, int32_t* pair_row, mxf_stream stream);

/*
 * moe_grouped_mxfp4_gemm - both expert FCs for every (token, expert) pair.
 * Defined by: page "DGX Spark 原生 FP4 矩阵指令" section 二 (the MoE MXFP4 entry;
 * weights stay FP4 into the matrix instruction), page "【DeepSeek V4】Triton FP4
 * 优化实战" sections "FP4 MoE GEMM 是什么？" (two FC per expert) and 第二步 (expert
 * FC1 is 4096 x 7168; even column in the low nibble), and page "Domestic GPUs are
 * awesome! ... DeepSeek-V4" ("SwiGLU + FP8 quant" fused between the two FCs).
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
 * moe_grouped_mxfp4_gemm_combine - both expert FCs with FC2 fused into the
 * gate-weighted combine, for decode-sized batches:
 *   out[t] = sum_{j=0..topk-1} gates[t][j] * (h_hat[r(t,j)] . W2_hat[e(t,j)]^T)
 * Defined by: the FC1 / SwiGLU / requantisation steps of moe_grouped_mxfp4_gemm
 * above, then the combine half of MoE dispatch/combine (page "Domestic GPUs are
 * awesome! ... DeepSeek-V4") applied inside the FC2 kernel, which the closing
 * lessons of page "【DeepSeek V4】Triton FP4 优化实战" motivate (cut the data moved
 * between steps, not the arithmetic). The FC2 products of one output column for
 * every (token, slot) pair stay in fp32 on the chip (y is never stored and never
 * rounded to bf16) and are summed in slot order j = 0, 1, ... with fused
 * multiply-adds, then stored as out_dtype (bf16: round to nearest even).
 *   q, q_scale, act_fmt, expert_offsets, sorted_pair, w1.., w2.., h, h_scale
 *                  as for moe_grouped_mxfp4_gemm (h is still written: FC2 reads it)
 *   topk_ids, pair_row, gates   [T][topk] int32, [T*topk] int32, [T][topk] fp32,
 *                  as written by moe_route_permute (FC1 reads the expert-grouped
 *                  order, the fused FC2 the token-major one)
 *   out            [T][H] fp32 or bf16 (out_dtype), caller-allocated
 * Requires T <= 64 (larger batches: moe_grouped_mxfp4_gemm + moe_unpermute_combine,
 * else UNSUPPORTED) and the shape rules of moe_grouped_mxfp4_gemm. Deterministic:
 * no atomics, fixed summation order. T == 0 is a no-op.
 * Errors: NULL, SHAPE, ALIGN, FORMAT, UNSUPPORTED.
 */
int moe_grouped_mxfp4_gemm_combine(const uint8_t* q, const uint8_t* q_scale, int act_fmt,
                                   int64_t T, int32_t topk, int64_t H, int64_t I, int32_t E,
                                   const int32_t* expert_offsets, const int32_t* sorted_pair,
                                   const int32_t* topk_ids, const int32_t* pair_row,
                                   const float* gates,
                                   const uint8_t* w1, const uint8_t* w1_scale,
                                   const uint8_t* w2, const uint8_t* w2_scale,
                                   uint8_t* h, uint8_t* h_scale,
                                   void* out, int out_dtype, mxf_stream stream);

/*
 * moe_unpermute_combine - out[t] = sum_{j=0..topk-1} gates[t][j] * y[pair_row[t*topk+j]]
 * Defined by: the combine half of MoE dispatch/combine, page "Domestic GPUs are
 * awesome! ... DeepSeek-V4"; the gates are the routing weights of page "【DeepSeek
 * V4】Triton FP4 优化实战" section "FP4 MoE GEMM 是什么？".
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

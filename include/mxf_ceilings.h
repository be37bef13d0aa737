/* Achievable-rate probes for MI355X (gfx950): measurement helpers beside the
 * expert-path calls of mxfp4_moe.h, not part of that path.
 *
 * A roofline fraction against a datasheet peak mixes two things: how close a
 * kernel comes to what the chip actually sustains, and how far that is from the
 * datasheet. These two calls measure what the chip sustains for the two bounds
 * the expert path runs into, and a third the prefill GEMMs' copies run into:
 *
 *   - mxf_ceiling_read: a streaming read of a device buffer with non-temporal
 *     16-byte loads that cover whole 128-byte lines (the HBM bound of the
 *     weight-streaming decode kernels);
 *   - mxf_ceiling_mfma: a register-only loop of 32x32x64 block-scaled MFMAs
 *     (V_MFMA_SCALE_F32_32X32X64_F8F6F4), E2M1 x E2M1 or E4M3 x E2M1, with
 *     operands taken from a caller buffer (the MFMA bound of the prefill GEMMs;
 *     random operand bits draw more power than constant ones and the chip lowers
 *     its clock accordingly, so the rate depends on the data);
 *   - mxf_ceiling_lds_copy: the HBM -> LDS copy path of the prefill GEMMs alone,
 *     with their stage size, lookahead and sharing of tiles between workgroups.
 *
 * Conventions as in mxfp4_moe.h: device pointers, asynchronous on the given
 * stream, arguments validated before anything is enqueued (status codes
 * MXF_OK / MXF_ERR_*), nothing allocated, cleared or synchronised.
 */
#ifndef MXF_CEILINGS_H
#define MXF_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#include "mxfp4_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of one mxf_ceiling_mfma launch (256 threads each: two per compute
 * unit of a 256-CU MI355X, i.e. two waves per SIMD) and the int32 operand words
 * it reads: 64 operand sets of 6 fragments x 64 lanes x 8 words; wave w of the
 * launch uses set w mod 64. */
#define MXF_CEILING_MFMA_GROUPS 512
#define MXF_CEILING_MFMA_WORDS (64 * 6 * 64 * 8)

/* Flops of one mxf_ceiling_mfma call with `iters` iterations:
 * 512 workgroups x 4 waves x iters x 8 MFMAs x 131,072 (2 x 32 x 32 x 64). */
int64_t mxf_ceiling_mfma_flops(int iters);

/* Run `iters` iterations of 8 independent 32x32x64 scaled MFMAs per wave.
 *   act_fmt   MXF_E2M1 (E2M1 x E2M1) or MXF_E4M3 (E4M3 x E2M1): the A operand's
 *             element format; B is always E2M1.
 *   operands  device, >= MXF_CEILING_MFMA_WORDS int32 words, 16-byte aligned:
 *             the operand bits (for E4M3 the lowest bit of every byte is cleared
 *             in registers, so no NaN code reaches the instruction).
 *   scale     the UE8M0 scale byte of both operands (127 = 2^0).
 *   iters     1 .. 1,000,000.
 *   sink      device, >= MXF_CEILING_MFMA_GROUPS floats, 16-byte aligned:
 *             workgroup g writes the sum of the 8 x 16 accumulator elements of
 *             its first lane. With every A and B element equal to 1.0 and scale
 *             127 each element is 64 x iters, so the sum is 8192 x iters, exact
 *             for iters <= 2048: that is how the loop is checked.
 * Errors: MXF_ERR_NULL, MXF_ERR_ALIGN, MXF_ERR_FORMAT, MXF_ERR_SHAPE (iters or
 * operand_words out of range), MXF_ERR_LAUNCH. */
int mxf_ceiling_mfma(int act_fmt, const int32_t* operands, int64_t operand_words, int scale, int iters,
                     float* sink, mxf_stream stream);

/* Read `bytes` bytes (a multiple of 16, 16-byte aligned) with non-temporal
 * 16-byte loads in a grid-stride loop (each wave reads 1 KB contiguous per
 * load instruction) and XOR every 32-bit word of the buffer into *xor_out with
 * one atomic per workgroup (*xor_out must hold the starting value, normally 0;
 * the result is the XOR of all words, which checks that every byte was read).
 * Errors: MXF_ERR_NULL, MXF_ERR_ALIGN, MXF_ERR_SHAPE, MXF_ERR_LAUNCH. */
int mxf_ceiling_read(const void* buf, int64_t bytes, int32_t* xor_out, mxf_stream stream);

/* The LDS-fill probe: the copy path of the 256 x 256 FP4 ring kernel on its own.
 * Workgroups of 512 threads (8 waves) hold 128 KB of LDS each (one per compute unit)
 * and fill it in MXF_CEILING_COPY_STAGES stages of 64 KB by HBM -> LDS copies
 * (buffer_load ... lds, 16 bytes per lane, 1 KB contiguous per instruction), one
 * stage ahead: after the wait and barrier that make stage s visible, the copies of
 * stage s + 1 go to the other half and every lane adds the 32-bit words of 128 bytes
 * of stage s (mod 2^32) into a running sum. Half of each stage comes from an
 * "activation" region, half from a "weight" region, each MXF_CEILING_COPY_REGION
 * bytes (the stages' 32 KB pieces in order).
 *   pattern 0: workgroup b reads activation region b and weight region groups + b:
 *              2 x groups regions, each read once (the copy path streaming HBM);
 *   pattern 1: the sharing of the grouped FC1 launch: block b = 8 j + x runs on XCD
 *              x; with j = 32 k + i, it reads activation region 2 (8 k + x) + i % 2
 *              (one per 256-row unit, shared by its 16 n-tiles) and weight region
 *              groups / 16 + 16 (8 k + x) + i / 2 (one per n-tile, shared by the
 *              unit's two workgroups): groups / 16 + groups / 2 regions.
 *   buf      device, 16-byte aligned, >= mxf_ceiling_lds_copy_bytes(pattern, groups)
 *            bytes (activation regions first, then weight regions).
 *   groups   workgroups, a positive multiple of 256, at most 65536.
 *   sum_out  device, 4-byte aligned: every workgroup adds its sum (one atomic per
 *            wave), so *sum_out gains the sum, mod 2^32, of every word each
 *            workgroup read: with pattern 1 each activation region counts 16 times
 *            and each weight region twice. That checks that every copy landed.
 * Errors: MXF_ERR_NULL, MXF_ERR_ALIGN, MXF_ERR_SHAPE (pattern, groups or bytes),
 * MXF_ERR_LAUNCH. */
#define MXF_CEILING_COPY_STAGES 28
#define MXF_CEILING_COPY_REGION (MXF_CEILING_COPY_STAGES * 32768)

/* Bytes the probe reads per workgroup (stages x 64 KB) is fixed; this returns the
 * buffer bytes a (pattern, groups) pair needs, or 0 when the pair is invalid. */
int64_t mxf_ceiling_lds_copy_bytes(int pattern, int groups);
int mxf_ceiling_lds_copy(const void* buf, int64_t bytes, int pattern, int groups, uint32_t* sum_out,
                         mxf_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MXF_CEILINGS_H */

/* attn_calib.h -- reference kernels for measurement, in libattn.so.
 *
 * They compute nothing of attention.  They measure what two plain kernels
 * reach on the GPU they run on: a streaming kernel that only reads and writes
 * HBM, and a loop of bf16 matrix-core instructions with no memory traffic.
 * A benchmark divides the attention kernels' rates by these rates to state
 * them as fractions of what is achievable on the part, next to the fractions
 * of the published peaks (8 TB/s HBM, 2.5 PFLOP/s dense bf16 MFMA).
 *
 * Same conventions as attn.h: device pointers, asynchronous on `stream`
 * (0 = the default stream), host-side validation before any launch (nothing
 * is launched or written on failure), status codes from attn.h.
 */
#ifndef ATTN_CALIB_H
#define ATTN_CALIB_H

#include <stddef.h>

#include "attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streams `src_bytes` from `src` and writes `dst_bytes` to `dst`.
 *   Chunk j (16 bytes) of dst = XOR of the 16-byte chunks j, j + n, j + 2n, ...
 *   of src, n = dst_bytes / 16.  So src_bytes == dst_bytes is a copy, and
 *   src_bytes = 3 * dst_bytes reads three streams per written one.  A small
 *   dst (a few MB) makes it a read-only stream; src_bytes == 0 writes zeros
 *   (a write-only stream, src may then be NULL).
 *   src, dst: device buffers, 16-byte aligned, not overlapping.
 * Errors: ATTN_ERR_NULL (null pointer with a nonzero size),
 *   ATTN_ERR_ARG (sizes not multiples of 16, src_bytes not a multiple of
 *   dst_bytes, dst_bytes == 0 with src_bytes > 0, or misaligned pointers),
 *   both sizes 0: nothing to do, ATTN_OK;
 *   ATTN_ERR_HIP (launch failure).  Bytes moved: src_bytes + dst_bytes. */
int attn_calib_stream(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                      hipStream_t stream);

/* Runs `iters` iterations of four independent v_mfma_f32_32x32x16_bf16 chains
 * in each of the 4 wavefronts of each of `workgroups` workgroups (operands in
 * registers, no memory traffic inside the loop), then writes one float per
 * wavefront to `out[workgroups * 4]` so the work cannot be dropped.
 * Work = attn_calib_mfma_flops(workgroups, iters) floating-point operations.
 * Errors: ATTN_ERR_NULL (out null with workgroups > 0), ATTN_ERR_ARG
 *   (workgroups or iters negative, or workgroups > 2^20), ATTN_ERR_HIP. */
int attn_calib_mfma(float* out, int workgroups, int iters, hipStream_t stream);

/* 2 * 32 * 32 * 16 flops per instruction * 4 chains * 4 wavefronts * iters * workgroups. */
double attn_calib_mfma_flops(int workgroups, int iters);

/* One v_mfma_scale_f32_32x32x64_f8f6f4 instruction (OCP E4M3 x E4M3 operands,
 * block scales 2^0, zero accumulator) on one wavefront:
 *     c[m][n] = sum_{k<64} e4m3(a[m][k]) * e4m3(b[n][k])   as the matrix core sums it.
 *   a, b: 32 x 64 byte codes, row-major (row m of a, row n of b hold the 64
 *         k-values); c: 32 x 32 fp32, row-major.  All 16-byte aligned.
 * The fp8 prefill computes its scores with this instruction; this call lets a
 * test observe the instruction's own accumulation error on constructed inputs.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_ARG (misaligned), ATTN_ERR_HIP. */
int attn_calib_mfma_fp8(const void* a, const void* b, float* c, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CALIB_H */

/*
 * attn_ceiling.h - C ABI of the ceiling microbenchmarks built into libattn.so.
 *
 * They measure, on the GPU that runs the attention kernels, the sustained
 * rates those kernels are bounded by, so that each kernel's achieved rate can
 * be reported against both the published MI355X peak and a measured one.
 * The tutorial page "Guide de programmation pour la programmation GPU par
 * tuiles de NVIDIA : de cuTile et des noyaux Triton a Flash Attention" times
 * each of its kernels against a reference; these probes give the reference
 * rates of the hardware units themselves (matrix cores, the exponential and
 * FMA vector ALUs, LDS reads, HBM).
 *
 * Conventions. Every pointer is a DEVICE pointer; the caller owns all memory.
 * Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and the
 * call returns without synchronising; the caller times it (HIP events on the
 * same stream). Return value: 0 on success, -1 for a bad argument (checked
 * before any HIP call), -3 if the launch reported an error.
 */
#ifndef ATTN_CEILING_H_
#define ATTN_CEILING_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * bf16 matrix-core rate: each wave runs `iters` iterations of 8
 * v_mfma_f32_32x32x16_bf16 (32768 FLOPs each) on 4 independent accumulators,
 * with 8 distinct (A, B) operand pairs held in registers.
 *   operands       device buffer of operand_lanes x 16 x 16 bytes (bf16); lane
 *                  g of the grid reads block g % operand_lanes (A[0..7], B[0..7],
 *                  8 bf16 each); 16-byte aligned
 *   out            workgroups x waves x 64 floats (written, a checksum)
 *   waves          4 or 8 waves per workgroup
 * FLOPs = workgroups * waves * iters * 8 * 32768.
 */
int attn_ceiling_mfma_bf16(const void* operands, int64_t operand_lanes, float* out,
                           int workgroups, int waves, int iters, void* stream);

/*
 * The same on v_mfma_f32_16x16x32_bf16: each wave runs `iters` iterations of
 * 16 of them (16384 FLOPs each) on 8 independent accumulators, from the same
 * operand buffer and with the same arguments as attn_ceiling_mfma_bf16.
 * FLOPs = workgroups * waves * iters * 16 * 16384.
 */
int attn_ceiling_mfma16_bf16(const void* operands, int64_t operand_lanes, float* out,
                             int workgroups, int waves, int iters, void* stream);

/*
 * Exponential rate: 256 threads per workgroup, 16 independent chains x <- 2^-x
 * per thread (one v_exp_f32 each). Exponentials = workgroups * 256 * iters * 16.
 *   out  workgroups x 256 floats (written)
 */
int attn_ceiling_exp2(float* out, int workgroups, int iters, void* stream);

/*
 * fp32 FMA rate (scalar v_fma_f32, no packed forms): 256 threads per workgroup,
 * 16 independent chains per thread. FMAs = workgroups * 256 * iters * 16.
 *   out  workgroups x 256 floats (written)
 */
int attn_ceiling_fma(float* out, int workgroups, int iters, void* stream);

/*
 * Exponentials and FMAs together: 256 threads per workgroup, 8 independent
 * exponential chains and 32 independent FMA chains per thread, one v_exp_f32
 * issued between every four v_fma_f32. Exponentials = workgroups * 256 * iters
 * * 8, FMAs = workgroups * 256 * iters * 32. Timed beside the two probes above,
 * it tells whether the exponential runs beside the FMAs (time = the larger
 * part) or takes their issue slots (time = the sum of the parts).
 *   out  workgroups x 256 floats (written)
 */
int attn_ceiling_exp2_fma(float* out, int workgroups, int iters, void* stream);

/*
 * LDS read bandwidth: 512 threads per workgroup (64 KiB of LDS each), 8 reads
 * per thread and iteration, bank-conflict-free. transposed = 0: ds_read_b128
 * (16 bytes per lane); transposed != 0: ds_read_b64_tr_b16 (8 bytes per lane).
 * Bytes = workgroups * 512 * iters * 8 * (16 or 8).
 *   out  workgroups x 512 floats (written)
 */
int attn_ceiling_lds_read(float* out, int workgroups, int iters, int transposed, void* stream);

/*
 * HBM copy: dst[0 .. bytes) = src[0 .. bytes), 16-byte accesses. bytes must be a
 * multiple of 16 and both pointers 16-byte aligned; the ranges must not overlap.
 * HBM traffic = 2 * bytes.
 */
int attn_ceiling_copy(void* dst, const void* src, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CEILING_H_ */

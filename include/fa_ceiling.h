/*
 * fa_ceiling.h -- C ABI of libfa_ceiling.so: measurement kernels that
 * show what MI355X (gfx950) sustains on the resources the attention
 * kernels of libfa_amd.so are bound by, so that their roofline fractions can
 * be read against an achievable ceiling as well as the published peak.
 * Nothing here is part of the attention path.
 *
 *  - The matrix-core ceiling: waves that do nothing but MFMAs of one shape
 *    (16x16x32 16-bit, the forward's; 32x32x16 16-bit, the backward's;
 *    32x32x64 FP8, the FP8 forward's) on operands taken from memory once,
 *    so the values the matrix cores multiply have the statistics of real
 *    inputs (power draw depends on them).
 *  - The LDS read ceiling: the operand reads of the attention kernels
 *    (16-byte row reads, 8-byte transposing reads) from a resident tile.
 *  - The HBM read ceiling: a grid-stride stream of 16-byte loads over a
 *    buffer much larger than the last-level cache, with the non-temporal
 *    policy the decode kernel uses, or the default one.
 *
 * All enqueue on `stream` and return hipSuccess (0) or the HIP error of the
 * launch; arguments are checked first (hipErrorInvalidValue, nothing
 * enqueued).  All pointers are device pointers owned by the caller.
 */
#ifndef FA_AMD_FA_CEILING_H
#define FA_AMD_FA_CEILING_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_ceiling_mfma -- `workgroups` workgroups of 4 waves; every wave issues
 * iters x 4 MFMAs in four independent accumulation chains:
 *   dtype 0: v_mfma_f32_32x32x16_bf16, 4 * 32768 * iters flops per wave
 *   dtype 1: v_mfma_f32_32x32x16_f16,  4 * 32768 * iters flops per wave
 *   dtype 2: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 (block scales 1),
 *            4 * 131072 * iters flops per wave
 *   dtype 3: v_mfma_f32_16x16x32_bf16, 4 * 16384 * iters flops per wave
 *   dtype 4: v_mfma_f32_16x16x32_f16,  4 * 16384 * iters flops per wave
 *   operands : each lane's A and B operand, 32 bytes per lane (dtypes 0, 1,
 *              3, 4) or 64 bytes per lane (dtype 2), workgroups * 256 lanes,
 *              16-byte aligned
 *   out      : workgroups * 256 floats (a checksum per lane, written)
 *   workgroups >= 1, iters >= 1
 */
int fa_ceiling_mfma(const void *operands, float *out, int workgroups, int iters, int dtype,
                    hipStream_t stream);

/*
 * fa_ceiling_lds -- LDS read bandwidth: `workgroups` workgroups of 4 waves,
 * each filling a 64 KiB LDS tile once and then reading it iters x 8 times per
 * lane, eight independent reads in flight:
 *   mode 0: ds_read_b128 (16 bytes per lane, 256 contiguous bytes per 16
 *           lanes): 128 bytes per lane per iteration
 *   mode 1: ds_read_b64_tr_b16 (8 bytes per lane): 64 bytes per lane per
 *           iteration
 *   out : workgroups * 256 uint32 (an XOR checksum per lane, written)
 *   workgroups >= 1, iters >= 1
 */
int fa_ceiling_lds(unsigned *out, int workgroups, int iters, int mode, hipStream_t stream);

/*
 * fa_ceiling_read -- reads `bytes` bytes of `src` once, 16 bytes per load:
 * workgroup w of `workgroups` (256 lanes each) streams the w-th contiguous
 * chunk of ceil(bytes / workgroups) bytes rounded up to 16 KiB;
 * nontemporal != 0 gives the loads the decode kernel's streaming
 * (non-temporal) cache policy.
 *   src : 16-byte aligned, bytes a positive multiple of 16, chunk < 2 GiB
 *   out : workgroups * 256 uint32 (an XOR checksum per lane, written)
 */
int fa_ceiling_read(const void *src, size_t bytes, unsigned *out, int workgroups,
                    int nontemporal, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_AMD_FA_CEILING_H */

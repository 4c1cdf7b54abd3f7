/*
 * sink_attn_peak.h -- achievable-peak probes of libsinkattn_peak.so, used by the
 * measurement harness beside the spec-sheet peaks (HBM 8 TB/s, dense bf16 MFMA
 * 2.5 PFLOP/s).  Not part of the attention library.  Device pointers, caller-owned;
 * work is enqueued on `stream` and nothing synchronises.  Return 0 on success, 1 for an
 * invalid argument, 4 if the launch failed.
 */
#ifndef SINK_ATTN_PEAK_H
#define SINK_ATTN_PEAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of buf[0, bytes) once with 16-byte non-temporal loads (the read
 * pattern of the decode kernels): num_blocks workgroups of 256 lanes, each streaming
 * one contiguous share of the buffer in order.
 * bytes a nonzero multiple of 16, buf 16-byte aligned; out4: 4 bytes of device memory
 * the kernel may write. */
int sink_attn_peak_stream_read(const void* buf, size_t bytes, int32_t num_blocks, void* out4,
                               void* stream);

/* num_blocks workgroups of 4 wavefronts, each wavefront issuing iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) from registers: num_blocks * 4 * iters * 8 *
 * 32768 flops.  out: num_blocks * 256 floats of device memory. */
int sink_attn_peak_mfma_bf16(int32_t iters, int32_t num_blocks, float* out, void* stream);

/* MFMA chains beside vector work: num_blocks workgroups, 4 wavefronts of each issuing
 * iters x 8 v_mfma_f32_32x32x16_bf16 as sink_attn_peak_mfma_bf16 does (num_blocks * 4 *
 * iters * 8 * 32768 flops), with pairs_per_mfma (0-4) pairs of one FMA and one exp2 per
 * MFMA: split = 0: issued by the MFMA wavefront itself after each MFMA (4 wavefronts a
 * workgroup, one per SIMD); split != 0: by a second wavefront on the same SIMD (8
 * wavefronts a workgroup).  out: num_blocks * 512 floats of device memory. */
int sink_attn_peak_coissue(int32_t pairs_per_mfma, int32_t split, int32_t iters,
                           int32_t num_blocks, float* out, void* stream);

/* Vector issue rate: num_blocks workgroups of 4 * waves_per_simd wavefronts (waves_per_simd
 * in {1, 2, 4}; one workgroup per CU fills every SIMD with that many), each wavefront
 * issuing iters x 8 independent instructions of one kind, op 0: v_exp_f32, op 1:
 * v_fma_f32 (num_blocks * 4 * waves_per_simd * iters * 8 wave64 instructions).
 * out: num_blocks * 256 * waves_per_simd floats of device memory; element 64 w of a
 * workgroup's 256 * waves_per_simd holds the shader-clock cycles wavefront w's loop took. */
int sink_attn_peak_valu(int32_t op, int32_t waves_per_simd, int32_t iters, int32_t num_blocks,
                        float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SINK_ATTN_PEAK_H */

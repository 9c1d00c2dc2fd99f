/*
 * qi_calib.h -- calibration microbenchmarks of the MI355X the library runs on.
 *
 * Roofline fractions are quoted against the vendor peaks and against what this
 * part measurably sustains: register-only MFMA throughput and a device copy.
 * These calls are diagnostics for the benchmark, not part of the DiT step: they
 * are exported by a separate, bench-only library, libqi_calib.so, and not by
 * libqi.so.  Unlike libqi, they allocate device memory, create a stream and
 * block until their measurement ends.
 */
#ifndef QI_CALIB_H_
#define QI_CALIB_H_

#include <stdint.h>

#include "qi.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Sustained bf16 MFMA throughput from a register-only loop on every CU:
 * shape 0 = v_mfma_f32_32x32x16_bf16, shape 1 = v_mfma_f32_16x16x32_bf16.
 * Runs `iters` iterations of 8 independent MFMA chains per wave on 8 workgroups
 * of 256 threads per CU, timed with HIP events on an internal stream, and
 * BLOCKS until done.  *tflops receives the result.  Errors: NULL, RANGE
 * (shape not 0/1, iters < 1), HIP. */
qi_status qi_calib_mfma_tflops(int32_t shape, int32_t iters, double *tflops);

/* Sustained device-to-device copy bandwidth (bytes read + written per second,
 * in GB/s) over `bytes` bytes (multiple of 16) between two caller buffers src
 * and dst (device, 16-byte aligned, not overlapping), best of `reps` timed
 * copies with HIP events, over grid-stride launches of 1024, 2048 and 4096
 * workgroups of 256 threads; BLOCKS until done.  Errors: NULL, RANGE, ALIGN, HIP. */
qi_status qi_calib_copy_gbs(const void *src, void *dst, int64_t bytes, int32_t reps, double *gbs);

/* Sustained read-only bandwidth (bytes read per second, GB/s) over `bytes`
 * bytes (multiple of 16) of src (device, 16-byte aligned), same launches and
 * timing as qi_calib_copy_gbs; scratch is a device buffer of at least
 * 4096 * 256 * 4 bytes that the kernel may write (it never does for real
 * data).  BLOCKS until done.  Errors: NULL, RANGE, ALIGN, HIP. */
qi_status qi_calib_read_gbs(const void *src, int64_t bytes, void *scratch, int32_t reps, double *gbs);

/* Shader cycles per iteration of a CU-wide LDS / MFMA instruction mix: one
 * workgroup of 512 threads (8 waves, two per SIMD, 128 KB of LDS) per CU, each
 * wave issuing per iteration
 *   mode 0: 8 ds_read_b128 (the GEMM's swizzled fragment reads),
 *   mode 1: 8 ds_write_b128 (the staging-store pattern),
 *   mode 2: 8 v_mfma_f32_32x32x16_bf16,
 *   mode 3: 8 MFMAs + 6 fragment reads + 2 staging stores (a register-staged
 *           GEMM K loop),
 *   mode 4: 8 MFMAs + 6 fragment reads + 2 16-byte-per-lane global -> LDS
 *           copies from a 64 KB buffer (a K loop fed by LDS copies),
 * with a barrier every fourth iteration, timed with the shader clock of wave
 * 0 of every workgroup and averaged.  Data are synthetic (values not used).
 * BLOCKS until done.  *cycles receives the cycles per iteration.  Errors:
 * NULL, RANGE (mode not 0..4, iters < 4), HIP. */
qi_status qi_calib_lds_cycles(int32_t mode, int32_t iters, double *cycles);

/* Wall-clock nanoseconds per iteration of a CU-wide VALU / MFMA instruction
 * mix, timed with HIP events over `iters` iterations on every CU (one
 * workgroup per CU); per iteration a wave issues 8 v_mfma_f32_32x32x16_bf16
 * and/or 32 VALU instructions on 8 independent register chains:
 *   mode 0: two waves per SIMD, each 32 v_exp_f32,
 *   mode 1: two waves per SIMD, each 32 v_fma_f32,
 *   mode 2: two waves per SIMD, each 8 MFMAs with the 32 v_exp_f32 of mode 0
 *           interleaved (four after each MFMA),
 *   mode 3: as mode 2 with the 32 v_fma_f32,
 *   mode 4: two waves per SIMD, each 8 MFMAs,
 *   mode 5: per SIMD one wave with the 8 MFMAs, the other with the 32
 *           v_exp_f32,
 *   mode 6: as mode 5 with the 32 v_fma_f32,
 *   mode 7: one wave per SIMD, 8 MFMAs,
 *   mode 8: one wave per SIMD, 32 v_exp_f32,
 *   mode 9: one wave per SIMD, 32 v_fma_f32.
 * Data are synthetic.  BLOCKS until done.  *ns receives the time per
 * iteration.  Errors: NULL, RANGE (mode not 0..9, iters < 4), HIP. */
qi_status qi_calib_valu_ns(int32_t mode, int32_t iters, double *ns);

#ifdef __cplusplus
}
#endif

#endif /* QI_CALIB_H_ */

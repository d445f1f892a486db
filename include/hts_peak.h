/*
 * hts_peak.h -- measured roofline denominators on AMD Instinct MI355X (gfx950), library
 * libhts_peak.so.  The hybrid product's throughput is reported as a fraction of the published
 * peaks (HBM 8 TB/s, dense 16-bit matrix cores 2.5 PFLOP/s) and of these measured ones: what one
 * streaming read reaches on this chip, and what the matrix-core instructions the product uses
 * deliver with their operands in registers (the sparse instruction of page "PATCH: Learnable
 * Tile-level Hybrid Sparsity for LLMs", section 2, inference and deployment: 2:4 tiles on the
 * sparse matrix cores, counted in kept multiply-adds).
 *
 * Every call is asynchronous on `stream` (a hipStream_t passed as void*, NULL = null stream); the
 * caller times it (events) and owns every buffer.  Returns 0, 1 for an invalid argument, or 8
 * when the launch failed.
 */
#ifndef HTS_PEAK_H
#define HTS_PEAK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (>= 16, 16-byte aligned device memory at src) once with `blocks` workgroups of 256
 * threads, 16-byte non-temporal loads, consecutive lanes on consecutive chunks.  sink: device
 * uint32, written only in a case no input reaches (keeps the loads). */
int hts_peak_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int blocks, void* stream);

/* Matrix-core throughput with register operands: `blocks` workgroups of 4 waves, each wave
 * `iters` rounds of 8 independent instructions of `kind`:
 *   0: v_mfma_f32_16x16x32_bf16      1: v_smfmac_f32_16x16x64_bf16 (2:4)
 *   2: v_mfma_f32_16x16x32_fp8_fp8   3: v_smfmac_f32_16x16x128_fp8_fp8 (2:4)
 *   4: v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 operands, unit scales)
 * out: device float[blocks * 256] (one value per thread, kept so the work is not removed). */
int hts_peak_mfma(int kind, int iters, int blocks, float* out, void* stream);

/* On-chip copy and read paths: `blocks` workgroups of 4 waves, each reading its own 64 KiB window
 * of src (window = workgroup index modulo bytes / 65536; keep bytes small enough to stay in L2,
 * e.g. 2 MiB) `iters` times, 16 bytes per lane:
 *   mode 0: global -> LDS by the direct copy (buffer load to LDS), the tiled product's copy path;
 *   mode 1: global -> registers;
 *   mode 2: LDS -> registers (16-byte LDS reads; src is not read).
 * Bytes moved = blocks x iters x 65536.  src: device memory of `bytes` >= 65536; sink as above. */
int hts_peak_onchip(int mode, const void* src, uint64_t bytes, int iters, int blocks, uint32_t* sink, void* stream);

/* Algorithmic flops of one instruction of `kind`: 2 x the multiply-adds of kept weights (a sparse
 * instruction keeps two of every four of its dense K); 0 for an unknown kind. */
double hts_peak_mfma_flops_per_instruction(int kind);

#ifdef __cplusplus
}
#endif

#endif /* HTS_PEAK_H */

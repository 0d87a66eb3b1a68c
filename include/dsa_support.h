/*
 * dsa_support.h -- measurement support for the dynamic sparse attention
 * library (libdsa.so): the chip's achievable ceilings, a cache flush, and a
 * probe of the FP8 matrix instruction.  Not part of the attention path.
 *
 * The pages ask that compute-bound and memory-bound stages be told apart and
 * profiled ([P5] "Day-0 Readiness for Trillion-Parameter Models: Engineering
 * Sparse Attention and Expert Weight Compression", "Verification and
 * Tuning").  These calls measure what MI355X sustains, so that a kernel's
 * rate can be quoted against both the published peak and the measured one.
 *
 * Conventions: device pointers owned by the caller; kernels are enqueued on
 * `stream` and nothing is synchronized.  Return 0 on success, -1 for a NULL
 * pointer or a size out of range, -3 for an unknown kind, -4 for a misaligned
 * pointer or size, -6 when HIP reports a launch error (text in
 * dsa_support_last_error(), thread-local).
 */
#ifndef DSA_SUPPORT_H
#define DSA_SUPPORT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads every byte of buf (bytes: a multiple of 16, buf 16 B aligned) once:
 * `grid` workgroups of 256 threads stride over it, each lane keeping four
 * independent 16 B loads in flight per step (variant 0: plain loads; 1:
 * non-temporal loads).  sink: uint32 [grid * 256], written (an XOR of the
 * data, so the reads cannot be dropped).  Time it with events on `stream`.
 */
int dsa_probe_stream_read(const void* buf, size_t bytes, int variant, unsigned* sink, int grid,
                          hipStream_t stream);

/*
 * Writes every 16 B of buf (bytes a multiple of 16, 16 B aligned), so that a
 * following kernel finds none of its inputs in the L2 or the last-level
 * cache when buf is larger than both.
 */
int dsa_cache_flush(void* buf, size_t bytes, unsigned seed, hipStream_t stream);

/*
 * Matrix-core rate: `grid` workgroups of four waves, each wave issuing
 * iters * 8 back-to-back MFMAs into eight independent accumulators, no memory
 * traffic.  Flops per MFMA: DSA_PROBE_MFMA_FP8 (v_mfma_scale_f32_16x16x128_f8f6f4,
 * E4M3 operands) 65536; DSA_PROBE_MFMA_I8 (v_mfma_i32_16x16x64_i8) 32768;
 * DSA_PROBE_MFMA_BF16 (v_mfma_f32_16x16x32_bf16) 16384.  sink: float
 * [grid * 256].
 */
enum { DSA_PROBE_MFMA_FP8 = 0, DSA_PROBE_MFMA_I8 = 1, DSA_PROBE_MFMA_BF16 = 2 };
int dsa_probe_mfma_rate(int kind, int iters, int grid, float* sink, hipStream_t stream);

/*
 * One v_mfma_scale_f32_16x16x128_f8f6f4 (E4M3 x E4M3, unit scales) per case:
 * d[c] = c_in[c] + A_c B_c, with a: uint8 [n_cases, 16 rows, 128] E4M3 codes,
 * b: uint8 [n_cases, 16 columns, 128] (column j of B stored as a row),
 * c_in, d: fp32 [n_cases, 16, 16] row-major.  a, b 16 B aligned.  The host
 * compares d with the exact sums to learn how the instruction accumulates.
 */
int dsa_probe_fp8_mfma(const uint8_t* a, const uint8_t* b, const float* c_in, int n_cases,
                       float* d, hipStream_t stream);

const char* dsa_support_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_SUPPORT_H */

/* Measured peaks of the chip (dense MFMA issue rate, HBM streaming rate), and a
 * register-fill test aid.
 *
 * A measurement aid that sits beside the attention library (libtsa_peaks.so,
 * built from the same tree): the attention kernels are compared against the
 * published peaks of the MI355X, and these kernels show what the same chip
 * sustains under the same clocks with nothing but back-to-back matrix
 * instructions, or nothing but coalesced 16-byte loads and stores.
 *
 * Every call only enqueues one kernel on `stream` (a hipStream_t, NULL for the
 * default stream) and returns; the caller times it with events on that stream.
 * Pointers are device pointers owned by the caller.  Return value: 0 on
 * success, -1 for an invalid argument (nothing launched), -2 when the launch
 * itself failed.
 */
#ifndef TSA_PEAKS_H
#define TSA_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n_blocks workgroups of 256 threads; every wave issues `iters` rounds of
 * four independent 32x32x16 MFMAs (dtype 0: bf16 inputs, 1: fp16 inputs,
 * fp32 accumulate) on operands whose every element is `a`.  out[blk]
 * (device, n_blocks floats) receives the sum of element 0 of the four
 * accumulators of the block's first wave: 64 * iters * a * a exactly when a*a
 * and the sums are representable.  *flops_out (host) receives the dense
 * FLOPs the launch performs: n_blocks * 4 waves * 4 * iters * 2*32*32*16.
 * Limits: 1 <= n_blocks <= 65536, 1 <= iters <= 1 << 20, dtype in {0, 1}. */
int tsa_peak_mfma(int dtype, int n_blocks, int iters, float a, float* out,
                  double* flops_out, void* stream);

/* dst[i] = src[i] for `bytes` bytes (a multiple of 16; both pointers 16-byte
 * aligned; the ranges must not overlap) with 16-byte vector loads and stores
 * over a grid-stride loop of n_blocks workgroups of 256 threads
 * (1 <= n_blocks <= 65536).  HBM traffic: 2 * bytes. */
int tsa_peak_copy(const void* src, void* dst, size_t bytes, int n_blocks, void* stream);

/* Reads `bytes` bytes (a multiple of 16, 16-byte aligned) with nontemporal
 * 16-byte vector loads over a grid-stride loop and writes, per workgroup, the xor of every
 * 32-bit word it read to out[blk] (device, n_blocks words).  HBM traffic:
 * bytes.  Limits as for tsa_peak_copy. */
int tsa_peak_read(const void* src, size_t bytes, int n_blocks, unsigned* out, void* stream);

/* As tsa_peak_read with plain (cached) loads: a buffer larger than the L2s
 * (4 MB per XCD) and smaller than the 256 MB memory-side cache (MALL), read
 * twice in a row, is then served from the MALL the second time. */
int tsa_peak_read_cached(const void* src, size_t bytes, int n_blocks, unsigned* out, void* stream);

/* Test aid: 4096 workgroups of 256 threads, one wave per SIMD at 512
 * registers each, write `pattern` into all 256 VGPRs and 256 AGPRs of their
 * wave.  A kernel launched next on the same device that reads a register it
 * never wrote then finds that pattern (say the bits of +inf or a NaN)
 * instead of whatever earlier work left, so such reads show in results. */
int tsa_fill_registers(unsigned pattern, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TSA_PEAKS_H */

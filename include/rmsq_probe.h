/*
 * rmsq_probe.h -- measurement aid shipped beside librmsq: a memory-only kernel that moves the
 * bytes of one fused residual add + RMSNorm + quantization launch (read x and the residual,
 * write the new residual, the codes and the scales) in the same row-to-thread layout, with no
 * arithmetic beyond an XOR that keeps every load live.  Its duration is the practical ceiling of
 * the memory system for that traffic; the fused kernel's duration over it says how much of the
 * gap to the HBM peak the kernel itself is responsible for.  librmsq_probe.so, C ABI; not part
 * of the op library.
 */
#ifndef RMSQ_PROBE_H
#define RMSQ_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define RMSQ_PROBE_API __attribute__((visibility("default")))
#else
#define RMSQ_PROBE_API
#endif

/*
 * rmsq_probe_stream -- one launch over `rows` rows of `hidden` bf16 elements.
 *  in0      [rows, hidden] 16-bit elements, read (required), 16-byte aligned.
 *  in1      [rows, hidden] 16-bit elements, read, or NULL.
 *  out0     [rows, hidden] 16-bit elements, written (in0 ^ in1 per 16-byte chunk), or NULL.
 *  out1     [rows, hidden * out1_bytes_per_chunk / 8] bytes, written, or NULL: per 8-element
 *           chunk, out1_bytes_per_chunk bytes (8: like FP8 codes, 4: like packed FP4 codes).
 *  out2     a scale-like stream, written, or NULL: out2_bytes (1 or 4; 4-byte aligned for 4)
 *           per 2^out2_shift chunks (0..6; the chunk count per row a multiple of it), stored by
 *           the thread holding the element's first chunk, [rows, hidden / 8 >> out2_shift]
 *           elements; out2_shift -1: one element per row (the thread of chunk 0).  Like the
 *           per-group (shift log2(G/8)), per-token (-1) and FP4 block (1, one byte) scales.
 *  threads_per_row, chunks_per_thread
 *           the fused kernel's launch shape: threads_per_row a multiple of 64 up to 1024,
 *           chunks_per_thread 1-8, threads_per_row * chunks_per_thread * 8 == hidden exactly;
 *           one workgroup per row, chunk c of a row on thread c mod threads_per_row.
 *  start_event, stop_event
 *           hipEvent_t or NULL: stamped by the dispatch itself (hipExtLaunchKernel).
 * Outputs must not overlap the inputs.  Returns 0, -1 for an invalid argument or shape, -2 for
 * a misaligned pointer, -5 if the launch failed.
 */
RMSQ_PROBE_API int rmsq_probe_stream(const void* in0, const void* in1, void* out0, void* out1,
                                     void* out2, int64_t rows, int64_t hidden,
                                     int out1_bytes_per_chunk, int out2_shift, int out2_bytes,
                                     int threads_per_row, int chunks_per_thread,
                                     void* start_event, void* stop_event, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RMSQ_PROBE_H */

/*
 * mdc_probe.h -- memory-ceiling probes (libmdc_probe.so) for AMD Instinct
 * MI355X (gfx950), used by the benchmark beside libmdc's kernels.
 *
 * None of these calls computes any part of the MoE method.  They move bytes in
 * the access patterns the dispatch and combine kernels use, with the same
 * wavefront shape and non-temporal loads and stores, so that a kernel's
 * duration can be compared with what the same bytes cost in the plainest
 * kernel of that pattern.  The pages name a measured comparison of the fused
 * operator but do not print it ("PTO MegaMoE Dispatch + Combine Fusion
 * Example", Measured Performance), so the ceilings are measured on the device.
 *
 * Conventions: device pointers owned by the caller, 16-byte aligned; sizes in
 * bytes are multiples of 16; work is enqueued on `stream` (a hipStream_t, NULL
 * = default stream) and the call returns at once.  Return value: 0 = enqueued,
 * 1 = the launch failed, 2 = a NULL pointer or a size that is not a positive
 * multiple of 16.  Row indices must lie inside the buffers they index: the
 * probes do not check them.
 */
#ifndef MDC_PROBE_H
#define MDC_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` from src (the words are folded; sink, 4 KiB, is written only
 * if the fold hits a fixed value, which keeps every load live). */
int mdc_probe_read(const void* src, uint64_t bytes, void* sink, void* stream);

/* Write `bytes` of a constant pattern to dst. */
int mdc_probe_write(void* dst, uint64_t bytes, uint32_t value, void* stream);

/* Copy `bytes` from src to dst. */
int mdc_probe_copy(const void* src, void* dst, uint64_t bytes, void* stream);

/* Read rows rows[0..n_rows) of src (row i starts at src + rows[i] * row_bytes),
 * two wavefronts per 14 KiB row: the dispatch gather's read half. */
int mdc_probe_rows_read(const void* src, const int32_t* rows, int32_t n_rows, int32_t row_bytes, void* sink,
                        void* stream);

/* For each source item i < n_src, write a constant to rows
 * rows[offsets[i] .. offsets[i+1]) of dst: the dispatch gather's token-major
 * fan-out write half (offsets holds n_src + 1 entries). */
int mdc_probe_rows_write(void* dst, const int32_t* offsets, const int32_t* rows, int32_t n_src, int32_t row_bytes,
                         void* stream);

/* For each source item i < n_src, read row src_rows[i] of src once and write it
 * to rows dst_rows[offsets[i] .. offsets[i+1]) of dst: the dispatch gather's
 * whole data movement (read once, token-major fan-out writes) without its
 * placement work. */
int mdc_probe_rows_fanout(const void* src, const int32_t* src_rows, const int32_t* offsets, const int32_t* dst_rows,
                          void* dst, int32_t n_src, int32_t row_bytes, void* stream);

/* For each output row t < n_out, read rows rows[t*k .. t*k + k) of src
 * (negative entries are absent) and row t of own, and write their XOR to row t
 * of dst: the combine's access pattern (k <= 16). */
int mdc_probe_rows_reduce(const void* src, const int32_t* rows, int32_t k, const void* own, void* dst, int32_t n_out,
                          int32_t row_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MDC_PROBE_H */

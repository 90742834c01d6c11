/*
 * q4_measure.h -- measurement entry points of libq4stream (MI355X, gfx950).
 *
 * Not part of the decode path: variants of the products with an explicit
 * launch shape, a kernel timer and copy timing for the weight stream, used
 * by the benchmark and the tests to compare implementations.  Conventions,
 * status codes and the weight format are those of q4.h.
 */
#ifndef Q4_MEASURE_H
#define Q4_MEASURE_H

#include "q4.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Tuning variants of the two products, for measurement: the same
 * arithmetic with an explicit launch shape.  q4_gemv_tuned: rows_per_slot
 * and k_split in {1, 2, 4} (rows held by each 16-lane row of a wave, waves
 * sharing one row's k range), chunks_in_flight in {2, 4, 8} (16-byte chunks
 * of each row a lane loads before using them; 2 selects the software-
 * pipelined loop, two register buffers of two chunks with the next batch
 * always in flight, which needs K % (1024 * k_split) == 0 and nontemporal 1,
 * else UNSUPPORTED; at equal rows_per_slot and k_split it gives the same
 * bits as the single-buffer loop), nontemporal 0/1 (weight loads marked
 * non-temporal).  q4_gemm_tuned: row_tiles in {1, 2, 4, 8} and
 * waves in {4, 8, 16} (16-row tiles per workgroup, waves splitting k), with
 * row_tiles 8 only for 4 waves and 4 only up to 8 waves; B == 1 is allowed
 * and runs the matrix-core kernel.
 * INVALID_ARG / UNSUPPORTED for other values. */
q4_status q4_gemv_tuned(const uint8_t *packed, const uint16_t *scales,
                        const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                        int32_t rows_per_slot, int32_t k_split, int32_t chunks_in_flight,
                        int32_t nontemporal, hipStream_t stream);
q4_status q4_gemm_tuned(const uint8_t *packed, const uint16_t *scales,
                        const uint16_t *X_f16, float *Y, int64_t N, int64_t K,
                        int32_t B, int32_t row_tiles, int32_t waves,
                        hipStream_t stream);

/* The row-per-wave batch-1 kernel that q4_gemv runs for K <= 4096 (all of
 * a lane's chunks in flight at once), with an explicit launch shape:
 * rows_per_wave 2 or 4 (rows a wave holds at a time), workgroups of four
 * waves (0: one group of rows per wave, capped at four workgroups per
 * compute unit).  Arguments as q4_gemv; the rows per wave and the grid do
 * not change any output's bits, which equal q4_gemv's.  UNSUPPORTED for
 * K > 4096, INVALID_ARG for other values. */
q4_status q4_gemv_rows_tuned(const uint8_t *packed, const uint16_t *scales,
                             const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                             int32_t rows_per_wave, int32_t workgroups, hipStream_t stream);

/* The phased row-per-wave batch-1 kernel that q4_gemv runs for K > 4096,
 * with an explicit launch shape: each wave takes rows_per_wave rows and
 * walks them in phases of chunks_per_phase 16-byte chunks per lane (rows 1
 * or 2 with 1, 2, 4 or 7 chunks; 4 rows with 2 or 4), the activation read
 * from LDS; workgroups as in q4_gemv_rows_tuned.  Any K up to Q4_MAX_K;
 * arguments as q4_gemv.  The launch shape does not change any output's
 * bits, which equal q4_gemv's (also for K <= 4096).  INVALID_ARG for other
 * values. */
q4_status q4_gemv_rowp_tuned(const uint8_t *packed, const uint16_t *scales,
                             const uint16_t *x_f16, float *y, int64_t N, int64_t K,
                             int32_t rows_per_wave, int32_t chunks_per_phase,
                             int32_t workgroups, hipStream_t stream);

/* Measurement variant: the vector-ALU batch kernel for B in {2, 3, 4, 8}
 * (4 and 8 only here: beyond three columns the library uses the matrix
 * cores),
 * arguments as q4_gemm_smallbatch; needs B * K * 2 <= 65536 (the columns
 * are staged in LDS).  UNSUPPORTED otherwise; every column equals q4_gemv
 * of that column bitwise. */
q4_status q4_gemm_valu(const uint8_t *packed, const uint16_t *scales,
                       const uint16_t *X_f16, float *Y, int64_t N, int64_t K,
                       int32_t B, hipStream_t stream);

/* Average duration in microseconds of one of the four kernels of a layer
 * (which: 0 QKV, 1 O, 2 gate+up, 3 down), launched `reps` times back to back
 * on `stream` between two timing events, cycling through the resident
 * layers so no launch rereads cached weights.  The O and down kernels add
 * into h on every launch: h is clobbered.  QKV is timed without attention.
 * Synchronises `stream`. */
q4_status q4_decode_kernel_time(void *dec, int32_t which, int32_t reps,
                                hipStream_t stream, float *avg_us);
/* Copy timing of a weight stream, for the overlap figure of the offload
 * mode.  After q4_wstream_set_timing(ws, capacity), each of the next
 * `capacity` weight_stream_begin calls records a timing event on the copy
 * stream(s) where its copy starts (after the wait for its slot to be free)
 * and one where it ends; capacity 0 turns timing off.  Creates events only;
 * INVALID_ARG for capacity < 0.  The stream must be idle when called. */
q4_status q4_wstream_set_timing(void *ws, int32_t capacity);
/* For every timed copy so far (at most `capacity`), its start and end in
 * milliseconds after the start of the first timed copy: host arrays
 * start_ms and end_ms; with two copy streams the earliest start and the
 * latest end of the two.  *n_out: how many.  Waits for the last timed copy
 * to end. */
q4_status q4_wstream_copy_times(void *ws, float *start_ms, float *end_ms,
                                int32_t capacity, int32_t *n_out);

#ifdef __cplusplus
}
#endif

#endif /* Q4_MEASURE_H */

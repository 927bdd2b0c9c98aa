/*
 * dsa_probes.h - measurement probes for MI355X, built as their own library (libdsa_probes.so).
 *
 * They compute nothing of the method.  They measure what the device reaches on the resources
 * the DSA path's kernels are priced against (bf16 MFMA issue, streaming HBM reads, random
 * 256-byte row gathers in the sparse attention's access pattern, and the float-atomic adds that
 * the attention backward scatters with), so that a kernel's fraction of a spec peak can be read
 * beside its fraction of an achievable one.  The benchmark is their only
 * user; the product library (dsa.h) does not depend on them.
 *
 * Conventions: device pointers; `stream` is a hipStream_t (NULL = default stream); each call
 * only enqueues work, so time it with events on that stream.  Sinks are written only in a case
 * the probes never produce (they keep the loads live).  Errors: DSA_PROBE_ERR_INVALID_ARG (checked
 * on the host, nothing enqueued) and DSA_PROBE_ERR_HIP (launch failed); the message of the last
 * failing call of this host thread is in dsa_probe_last_error().
 */
#ifndef DSA_PROBES_H
#define DSA_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_PROBE_OK 0
#define DSA_PROBE_ERR_INVALID_ARG 1
#define DSA_PROBE_ERR_HIP 4

const char* dsa_probe_last_error(void);

/*
 * `grid` workgroups of four waves, each running `iters` iterations of eight independent
 * 16x16x32 (shape 16, the prefill indexer's instruction) or four 32x32x16 (shape 32) bf16 MFMA
 * chains with operands in registers.  sink [grid] float.  *flops (host, may be NULL) receives
 * the floating-point operations one call executes.  Grid in [1, 2^20], iters >= 1.
 */
int dsa_probe_mfma_bf16(int shape, int grid, int iters, float* sink, long long* flops, void* stream);

/*
 * Reads `bytes` of src (16-byte aligned, a positive multiple of 16) once with 16-byte loads from
 * `grid` workgroups of 256 threads, grid-stride.  sink [grid] uint32.
 */
int dsa_probe_stream_read(const void* src, size_t bytes, int grid, uint32_t* sink, void* stream);

/*
 * The memory traffic of the sparse GQA attention with no arithmetic: one wave per (row, KV
 * group g, split) reads, for every index entry p >= 0 of its row (idx [rows, k_sel] int32, the
 * row's entries split into nsplit ranges of 32-entry chunks), the key row and the value row
 * k[P, g, :], v[P, g, :] with P = row * row_stride + p (256 bytes each; P >= n_pos reads row 0),
 * with 16-byte loads and `depth` (1, 2 or 4) chunks of 32 entries in flight.  Load shape:
 * whole_rows = 0 reads as the per-row attention kernel does (each lane 64 contiguous bytes of one
 * entry's row, 16 rows per instruction); whole_rows = 1 lets 16 lanes read one whole 256-byte row
 * (4 rows per instruction, the shape of the kernels' row copies into LDS).  Work order: KV group
 * slowest (group_fastest = 0, the prefill kernels') or fastest (the decode kernel's).
 * k, v [n_pos, hkv, 128] bf16, 16-byte aligned.  sink [sink_len] uint32 with sink_len >= the
 * number of workgroups, ceil(rows * hkv * nsplit / 4) rounded up to 8.
 */
int dsa_probe_gather(const void* k, const void* v, int64_t n_pos, int hkv, const int32_t* idx, int k_sel, int rows,
                     int nsplit, int64_t row_stride, int group_fastest, int depth, int whole_rows, uint32_t* sink,
                     int64_t sink_len, void* stream);

/*
 * Float-atomic throughput in the shapes the attention backward scatters dk / dv with: `grid`
 * workgroups of four waves, each wave running `iters` atomic adds of 1.0 at 64 addresses, which
 * lie in 64 / floats_per_row rows of 128 floats (pseudo-random rows in [0, n_rows)) with
 * floats_per_row (16 or 64) consecutive floats in each.  buf [n_rows, 128] float (accumulates:
 * zero it first to check the count).  *adds (host, may be NULL) receives the additions one call
 * makes.  n_rows in [1, 2^32], grid in [1, 2^20], iters >= 1.
 */
int dsa_probe_atomic_add(float* buf, int64_t n_rows, int floats_per_row, int grid, int iters, long long* adds,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_PROBES_H */

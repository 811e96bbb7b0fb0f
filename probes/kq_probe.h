/*
 * kq_probe.h -- measurement probes that give the kq kernels' rooflines an
 * "achievable" denominator on the machine at hand, beside the MI355X
 * datasheet peaks (HBM 8.0 TB/s, dense int8 MFMA 5.0 POP/s).  They are not
 * part of the matmul; they exist so a benchmark can say how close a kernel
 * runs to what the same hardware reaches on the simplest code of its kind.
 *
 * Conventions as in kq.h: device pointers owned by the caller, `stream` a
 * hipStream_t as void*, everything checked on the host before any launch,
 * status codes KQ_OK / KQ_EINVAL / KQ_EALIGN / KQ_ELAUNCH.
 */
#ifndef KQ_PROBE_H
#define KQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility push(default)
#endif

/* Streaming read: `grid` workgroups of 256 threads read the `bytes` bytes at
 * `buf` once with 16-byte loads (grid-strided, four loads in flight per
 * thread) and fold them into an xor that is stored to `sink` (4 bytes) only
 * if it equals a value no ordinary buffer produces -- the store keeps the
 * loads live.  The read rate of a weight-sized buffer is the ceiling a
 * bandwidth-bound GEMV over the same bytes can approach.
 * buf: 16-byte aligned, bytes a positive multiple of 16; 1 <= grid <= 65536. */
int kq_probe_read(const void *buf, size_t bytes, uint32_t *sink, int grid, void *stream);

/* kq_probe_read with `unroll` (1, 2, 4, 8 or 16) loads in flight per thread
 * instead of four; the sweep over unroll, grid and size finds the best
 * plain read this machine sustains for a given buffer size. */
int kq_probe_read_u(const void *buf, size_t bytes, uint32_t *sink, int grid, int unroll, void *stream);

/* Matrix-core rate: `grid` workgroups of 256 threads; every wave issues
 * `iters` x 4 independent v_mfma_i32_32x32x32_i8 on register operands
 * (65,536 int8 ops each) and each thread stores one int of the results to
 * sink[grid * 256] so none is dead.  Ops per launch =
 * grid * 4 * iters * 4 * 65536.  1 <= grid <= 65536, 1 <= iters <= 2^24. */
int kq_probe_mfma_i8(int64_t iters, int grid, int32_t *sink, void *stream);

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif

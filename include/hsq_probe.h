/*
 * hsq_probe.h -- C ABI of libhsq_probe: measurement kernels for the MI355X
 * (gfx950) that give the layer's kernels their measured ceilings.  They are
 * not part of the layer and compute nothing of the method; bench.py
 * --probe times them with HIP events on the stream they are enqueued on.
 *
 * Conventions: device pointers, 16-byte aligned, owned by the caller;
 * `stream` is a hipStream_t passed as void*; every call only enqueues and
 * returns HSQ_OK (0) or a negative HSQ_E_* code of hsq.h (-1: bad argument,
 * -3: misaligned pointer, -5: launch refused).  Nothing is allocated.
 */
#ifndef HSQ_PROBE_H
#define HSQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Loop bodies of the int8 MFMA probe.  Each wave keeps the residual
 * contraction's wave tile (4 x 2 tiles of v_mfma_i32_16x16x64_i8, register
 * operands) and runs `iters` steps of 8 MFMAs; the modes add, per MFMA
 * result element and step, the contraction's VALU work on the previous
 * step's results:
 *   HSQ_PROBE_MFMA        MFMAs only (the matrix core's own rate)
 *   HSQ_PROBE_MFMA_FMA1   + 1 fp32 FMA per element
 *   HSQ_PROBE_MFMA_FMA2   + 2 fp32 FMAs per element (the exact rescale:
 *                         u = fma(D, sw, c), acc = fma(u, sx, acc))
 *   HSQ_PROBE_MFMA_FMA2_LDS  + the per-step LDS operand reads of the tiled
 *                         contraction (4 A and 2 B 16-byte reads per lane,
 *                         weight and activation scales)
 *   HSQ_PROBE_WIDE_FMA2, HSQ_PROBE_WIDE_FMA2_LDS  the FMA2 and FMA2_LDS
 *                         bodies with a wave tile of 4 x 4 MFMA tiles
 *                         (64 x 64 outputs: 16 MFMAs per step, 4 B reads) */
#define HSQ_PROBE_MFMA          0
#define HSQ_PROBE_MFMA_FMA1     1
#define HSQ_PROBE_MFMA_FMA2     2
#define HSQ_PROBE_MFMA_FMA2_LDS 3
#define HSQ_PROBE_WIDE_FMA2     4
#define HSQ_PROBE_WIDE_FMA2_LDS 5

/* Enqueue the MFMA probe: `blocks` workgroups of `waves` waves (1..16; at
 * most 8 for the wide modes) each; every wave runs `iters` steps (8 MFMAs
 * of 16*16*64 multiply-adds each, 16 for the wide modes).  out: blocks *
 * waves * 64 int32, written so the work is not optimised away. */
int hsq_probe_mfma(int mode, int iters, int blocks, int waves, int32_t *out, void *stream);

/* Stream probes over `bytes` bytes (a multiple of 16):
 *   hsq_probe_read: every byte of src read once with 16-byte loads (grid of
 *     `blocks` workgroups of 256 threads striding over the buffer); one
 *     int32 per thread written to sink (blocks * 256 int32).
 *   hsq_probe_copy: dst = src with 16-byte loads and stores. */
int hsq_probe_read(const void *src, size_t bytes, int blocks, int32_t *sink, void *stream);
int hsq_probe_copy(const void *src, size_t bytes, int blocks, void *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* HSQ_PROBE_H */

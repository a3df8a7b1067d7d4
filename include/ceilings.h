/*
 * ceilings.h -- C ABI of libceilings.so: machine-ceiling kernels the
 * benchmark measures beside the LoRA path, so each result can be reported as
 * a fraction of what this GPU sustains for the same kind of work (the
 * measurement method of the fast_trimul page, section "Benchmark": results
 * against machine ceilings), not only of the datasheet figures.
 *
 * Not part of the LoRA path.  All pointers are DEVICE pointers owned by the
 * caller; work is enqueued on `stream` (hipStream_t as void*, NULL = null
 * stream) without synchronising.  Return 0 on launch, 1 on a bad argument,
 * 4 on a misaligned pointer, 8 on a HIP launch error; nothing is launched on
 * an error.
 */
#ifndef RG_CEILINGS_H
#define RG_CEILINGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 MFMA loop: `workgroups` x `waves` (1..8) waves, each running
 * `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 on register
 * operands.  out: workgroups * waves * 64 floats (results, kept so the work
 * is not removed).  clocks: workgroups * 4 uint64 per launch: the shader
 * clock counter (s_memtime) at the first wave's start and end, then the
 * 100 MHz real-time counter (s_memrealtime) at the same two points; the
 * ratio of their spans times 100 MHz is the clock the work ran at. */
int ceil_mfma(int workgroups, int waves, int iters, float *out, uint64_t *clocks, void *stream);

/* Flops one ceil_mfma launch performs. */
double ceil_mfma_flops(int workgroups, int waves, int iters);

/* dst[0, bytes) = src[0, bytes): a streaming copy, 16 B per lane, 256-lane
 * workgroups.  variant 0: every lane strides over the whole buffer, four
 * loads in flight; 1: each workgroup streams one contiguous block, eight
 * 4-KiB rounds in flight; 2: as 1 with non-temporal loads and stores.
 * bytes a multiple of 16, pointers 16-byte aligned, buffers not
 * overlapping. */
int ceil_copy(const void *src, void *dst, int64_t bytes, int workgroups, int variant,
              void *stream);

/* Reads src[0, bytes) (16 B per lane, variants as ceil_copy) and writes
 * nothing unless every word of a lane's XOR of its data is all ones; out:
 * `workgroups` uint32 the kernel may write in that case.  bytes a multiple
 * of 16, src 16-byte aligned. */
int ceil_read(const void *src, int64_t bytes, void *out, int workgroups, int variant,
              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RG_CEILINGS_H */

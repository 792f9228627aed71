/*
 * fa_probe.h — measurement probes for the roofline of the attention kernels (AMD
 * Instinct MI355X, gfx950). Not needed to compute attention.
 *
 * The page "编译器与内核" (Compilers and kernels), section "屋顶线是上界，不是秒表", bounds
 * a kernel's throughput by min(P_max, B_max * I): P_max must belong to the same dtype and
 * instruction path as the kernel's FLOP count, and B_max is best measured for the access
 * pattern rather than taken from a specification sheet. These calls launch one probe
 * kernel each, asynchronously on `stream` (NULL = the default stream); the caller times
 * them (for example with events on the same stream) and divides.
 */
#ifndef FA_PROBE_H_
#define FA_PROBE_H_

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_probe_copy — copies `bytes` bytes from src to dst (device pointers, caller-owned,
 * 16-byte aligned, bytes a positive multiple of 16, not overlapping) with 16-byte loads
 * and stores. With buffers far larger than the last-level cache, 2 * bytes / time is the
 * streaming HBM bandwidth B_max. Returns FA_OK, FA_ERR_NULL for invalid arguments,
 * FA_ERR_DEVICE or FA_ERR_LAUNCH.
 */
int fa_probe_copy(const void* src, void* dst, int64_t bytes, void* stream);

/*
 * fa_probe_mfma — `blocks` workgroups of four waves, each wave running `iters` rounds of
 * four independent v_mfma_f32_32x32x16_bf16 chains on register operands (two
 * workgroups per compute unit fit, as in the attention kernel); writes blocks * 256
 * floats to out (caller-owned device memory) so the chains are kept. Its FLOP count is
 * fa_probe_mfma_flops(blocks, iters); FLOPs / time is the bf16 matrix-core ceiling
 * P_max at the clock the device sustains under that load. Returns FA_OK, FA_ERR_NULL or
 * FA_ERR_LAUNCH.
 */
int fa_probe_mfma(float* out, int blocks, int iters, void* stream);

/* The FLOPs one fa_probe_mfma launch performs: blocks * 4 waves * iters * 4 * 32768. */
double fa_probe_mfma_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */

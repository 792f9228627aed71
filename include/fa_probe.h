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
 * fa_probe_read — reads `bytes` bytes at src (device memory, 16-byte aligned, bytes a
 * positive multiple of 16) with 16-byte loads, four in flight per lane, and writes one word
 * per workgroup to sink (device memory, caller-owned, sink_words >= the grid: at most
 * 16 * the CU count). With a buffer far larger than the last-level cache, bytes / time is
 * the HBM read bandwidth, the B_max of kernels that mostly read (a decoding step, a bias
 * stream). Returns FA_OK, FA_ERR_NULL, FA_ERR_SHAPE (sink too small), FA_ERR_DEVICE or
 * FA_ERR_LAUNCH.
 */
int fa_probe_read(const void* src, int64_t bytes, unsigned* sink, int sink_words, void* stream);

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

/*
 * fa_probe_issue — how one SIMD's matrix core and vector ALU share instruction streams
 * (the steady state of the attention kernels interleaves MFMAs with the softmax's vector
 * work). Launches `blocks` workgroups; each "MFMA wave" runs `iters` rounds of two
 * alternating accumulator chains of v_mfma_f32_32x32x16_bf16 with `valu_ops` independent
 * v_fma_f32 and `exps` independent v_exp_f32 after each MFMA; each "VALU wave" runs
 * `iters` steps of 12 independent v_fma_f32 (or 4 v_exp_f32 when exps > 0).
 *   role 0: 4-wave workgroups (one wave per SIMD), all MFMA waves; valu_ops in
 *           {0, 2, 4, 6, 8, 12} with exps 0, or valu_ops 0 with exps in {1, 2, 4}, or
 *           valu_ops 4 with exps in {1, 2};
 *   role 1: 8-wave workgroups (waves w and w + 4 share a SIMD), waves 0-3 MFMA, 4-7 VALU;
 *   role 2: the same workgroups, only waves 0-3 working; role 3: only waves 4-7 working;
 *   role 4: all eight waves VALU waves (two per SIMD); valu_ops must be 0 for roles 1-4.
 * Writes blocks * threads floats to out and, per wave i, ticks[2i] = s_memtime cycles (the
 * shader clock) and ticks[2i+1] = s_memrealtime ticks (100 MHz) of its loop, 0 for idle
 * waves (device memory, caller-owned, 2 * blocks * 8 entries). Returns FA_OK, FA_ERR_NULL,
 * FA_ERR_SHAPE for an unsupported (valu_ops, exps) or FA_ERR_LAUNCH.
 */
int fa_probe_issue(int role, int valu_ops, int exps, int blocks, int iters, float* out, long long* ticks,
                   void* stream);

/*
 * fa_probe_lds — LDS throughput of one access kind. `blocks` workgroups of four waves, 64 KiB
 * of LDS each (two per compute unit); each wave runs `iters` rounds of eight accesses at
 * consecutive per-lane addresses (free of bank conflicts). mode: 0 ds_read_b128 (16 bytes
 * per lane), 1 ds_read_b64 (8), 2 ds_read_b64_tr_b16 (8, the transposing read of the V
 * operand), 3 ds_read_b32 (4), 4 ds_write_b128 (16, each round ends with a wait for its
 * writes). A wave moves iters * 8 * 64 * (bytes per lane) bytes. Writes blocks * 256 words
 * to out and, per wave i, ticks[2i] = s_memtime cycles and ticks[2i+1] = s_memrealtime ticks
 * (100 MHz) of its loop (device memory, caller-owned, 2 * blocks * 4 entries). Returns
 * FA_OK, FA_ERR_NULL, FA_ERR_SHAPE (unknown mode) or FA_ERR_LAUNCH.
 */
int fa_probe_lds(int mode, int blocks, int iters, unsigned* out, long long* ticks, void* stream);

/*
 * fa_probe_tile — a model of the forward kernel's steady-state tile body (the loop that
 * streams K and V tiles past a resident Q tile): its instruction mix without its data
 * dependences. `blocks` workgroups of four waves, two per compute unit, 64 KiB of LDS
 * each; per tile and wave, 32 MFMA slots (16 whose A operand takes two ds_read_b64_tr_b16,
 * 16 whose A operand takes one ds_read_b128, the reads three slots ahead), valu_ops
 * independent v_fma_f32 (0 or 117) and 33 independent v_exp_f32, and one workgroup barrier.
 * copies = 1 adds the kernel's tile copies: per wave and tile, after a wait for its earlier
 * copies and the barrier, eight 1 KiB LDS-DMA loads from the first 256 KiB at src (device
 * memory, 16-byte aligned, src_bytes >= 262144; it stays in the L2 cache); copies = 0
 * ignores src. Writes blocks * 256 floats to out and per-wave loop times to ticks as
 * fa_probe_lds does; a wave's cycles / tiles is the cycles per tile of its SIMD's pair of
 * waves. Returns FA_OK, FA_ERR_NULL, FA_ERR_SHAPE (copies not 0 or 1, valu_ops not 0 or
 * 117, src too small or misaligned) or FA_ERR_LAUNCH.
 */
int fa_probe_tile(int copies, int valu_ops, int blocks, int tiles, const void* src, int64_t src_bytes, float* out,
                  long long* ticks, void* stream);

/* Most launches one fa_probe_timer_arm call can arm. */
#define FA_PROBE_TIMER_MAX 4096

/*
 * fa_probe_timer_arm — arms kernel-timestamp timing for the next n launches, made by the
 * calling thread, of the main attention kernels (the forward kernel of fa_fwd, fa_fwd_qk
 * and their variants, and the dK/dV/dQ kernel of fa_bwd; not the merge, row-statistics or
 * reduction kernels). Each such launch then goes through hipExtLaunchKernelGGL with its
 * own pair of events, which the kernel's dispatch stamps at its start and at its end, so
 * the time excludes the host and queue gaps around the launch (the same interval a
 * kernel-trace profiler reports). The events are created by the library on the device
 * current at this call (a grow-only pool per thread, released at process end, or when the
 * thread arms the timer on another device); the armed launches must be made on that
 * device. Arming again drops the pairs not yet read; n = 0 disarms. 0 <= n <=
 * FA_PROBE_TIMER_MAX, else FA_ERR_NULL; FA_ERR_DEVICE if an event cannot be created. The
 * launches compute the same results; they cost a little more (the events add work between
 * consecutive kernels), so a measured step should not be armed. Not for launches made
 * while the stream is being captured into a graph.
 */
int fa_probe_timer_arm(int n);

/*
 * fa_probe_timer_read — waits for the armed launches and writes the duration of each, in
 * microseconds, in launch order, to us[0 .. n-1] (host memory, caller-owned); n must
 * equal the number of armed launches made since fa_probe_timer_arm (else FA_ERR_NULL).
 * Disarms the timer. FA_ERR_DEVICE if the events cannot be read.
 */
int fa_probe_timer_read(float* us, int n);

#ifdef __cplusplus
}
#endif

#endif /* FA_PROBE_H_ */

/*
 * fa_bwd.h — C ABI of the gradients of the exact attention forward (include/fa.h) for
 * AMD Instinct MI355X (gfx950).
 *
 * The page "编译器与内核" (Compilers and kernels), section "FlashAttention 围绕 IO 改写算法",
 * says the backward pass can recompute the score and probability blocks instead of
 * storing them. This library does exactly that: from Q, K, V, the forward's output O
 * and log-sum-exp, and the upstream gradient dO it forms, block by block,
 *
 *     P_ij = exp(S_ij - lse_i),   D_i = dO_i . O_i,
 *     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),
 *     dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d),
 *
 * the chain rule of the forward definition S = Q K^T / sqrt(d) + C, P = rowsoftmax(S),
 * O = P V (the pages print the method, not these formulas). S and P never reach device
 * memory. C (the bias and the causal mask, with the same conventions as fa_fwd) is a
 * constant: no gradient is formed for it. A query row with no allowed key (lse = -inf)
 * gets dQ = 0 and adds nothing to dK, dV.
 *
 * Numerics: bf16 or fp16 (all of q, k, v, out, grad_out and the gradients in the same
 * dtype). Products run on the matrix cores with fp32 accumulation; P and dS are rounded
 * to that dtype as operands; D uses the O it is given; dQ, dK, dV are rounded once. Every sum is formed in a fixed order inside one workgroup: for
 * a fixed build, device, shape and input, results are bitwise reproducible.
 */
#ifndef FA_BWD_H_
#define FA_BWD_H_

#include <stddef.h>
#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Element strides (not bytes) of every tensor, as in fa_strides. The innermost axis of
 * each is contiguous: d for q, k, grad_q, grad_k; dv for v, out, grad_out, grad_v; the
 * key axis for the bias; n for lse. Inputs may use stride 0 to broadcast. */
typedef struct {
  int64_t q[3], k[3], v[3];       /* [b, h, n] strides of the forward inputs           */
  int64_t out[3], grad_out[3];    /* O of the forward and the upstream gradient dO      */
  int64_t grad_q[3], grad_k[3], grad_v[3]; /* outputs                                  */
  int64_t bias[3];                /* bias[b, h, i, :] at bias + b*s0 + h*s1 + i*s2      */
  int64_t lse[2];                 /* lse[b, h, :] at lse + b*s0 + h*s1                  */
} fa_bwd_strides;

/*
 * fa_bwd — gradients of fa_fwd, enqueued on `stream`.
 *
 * q, k, v, bias, mask_mode, B, H, N, d, dv: exactly as given to fa_fwd.
 * out, lse: the forward's O ([B, H, N, dv], dtype) and log-sum-exp ([B, H, N], fp32).
 * grad_out: dO, [B, H, N, dv] in dtype.
 * grad_q, grad_k: [B, H, N, d]; grad_v: [B, H, N, dv]; dtype; fully written.
 * strides: NULL means contiguous [B, H, N, *] tensors, [B, H, N, N] bias, [B, H, N] lse.
 * dtype: FA_BF16 or FA_F16 (FA_F32 returns FA_ERR_DTYPE); d, dv: 64 or 128.
 * Alignment: every 16-bit tensor base and non-zero stride 16-byte aligned; bias and lse
 * 4-byte aligned. grad_q, grad_k, grad_v must not overlap any input or each other.
 * Workspace: fa_bwd_workspace_size() bytes (the authority): 8 bytes of row statistics
 * per row (rounded up to 128 rows per (b, h)) and, for problems with few tiles whose
 * loops are cut into chunks, fp32 partial sums of every chunk unit: units_kv * 128 *
 * (d + dv) plus units_q * 128 * d floats (tens of MiB for one long head). fa_bwd takes
 * it from the library-owned buffer of (device, stream) that fa_fwd also uses (include/
 * fa.h: calls on one stream run in order; the buffer only grows and old buffers stay
 * allocated until fa_shutdown()). While `stream` captures a graph, fa_bwd returns
 * FA_ERR_WORKSPACE: captured work takes fa_bwd_ex.
 * Returns FA_OK or a negative fa_status; validation happens before any launch, and a
 * failed call launches nothing. Asynchronous.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
           const void* grad_out, const float* bias, int mask_mode, void* grad_q, void* grad_k,
           void* grad_v, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
           const fa_bwd_strides* strides, int dtype, void* stream);

/* Bytes of scratch memory fa_bwd_ex needs (0 for invalid arguments or B*H*N == 0); the
 * workspace contract of the page "编译器与内核", section "生态系统也是目标的一部分". */
size_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype,
                             int mask_mode);

/* fa_bwd with caller-provided scratch memory (256-byte aligned, at least
 * fa_bwd_workspace_size bytes, no initialisation needed); allocates nothing and is safe
 * under graph capture. Same method and numerics as fa_bwd. */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* out, const float* lse,
              const void* grad_out, const float* bias, int mask_mode, void* grad_q, void* grad_k,
              void* grad_v, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
              const fa_bwd_strides* strides, int dtype, void* stream, void* workspace,
              size_t workspace_bytes);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H_ */

/*
 * fa.h — C ABI of the exact scaled-dot-product attention forward for AMD Instinct
 * MI355X (gfx950).
 *
 * The operation is the one defined on the page "编译器与内核" (Compilers and
 * kernels), section "FlashAttention 围绕 IO 改写算法", first display equation: for
 * every batch b and head h,
 *
 *     S = Q K^T / sqrt(d) + C,    P = row-softmax(S),    O = P V,
 *
 * with Q, K of shape N x d, V of shape N x dv, and C an additive bias/mask in which
 * -inf forbids a key. The library evaluates it with the online-softmax recurrence
 * of the same section (running max m_t, rescale alpha_t = exp(m_{t-1} - m_t),
 * running normaliser l_t and numerator o_t, O_i = o_T / l_T), so the N x N score and
 * probability matrices never reach device memory. It also returns the per-row
 * log-sum-exp  lse_i = m_i + ln(l_i) = ln sum_j exp(S_ij)  (natural log).
 *
 * C is the sum of (a) the optional fp32 bias tensor and (b) the causal mask
 * (C_ij = -inf for key j > query i + (N_k - N_q); for the square problems of fa_fwd,
 * N_q = N_k = N and this is the mask above the diagonal) when
 * mask_mode == FA_MASK_CAUSAL. The scale is 1/sqrt(d) with d the Q/K width, also
 * when d != dv. The bias is added after scaling and is not scaled.
 *
 * fa_fwd_qk takes N_q query rows against N_k keys (the pages treat N_q = N_k = N and
 * fix no causal convention for other lengths; this library aligns the query rows to
 * the end of the key sequence: query i is position N_k - N_q + i, so a single query
 * row sees every key, as in decoding against a key/value cache).
 *
 * The page assumes every query row has at least one allowed key. For a row that has
 * none, this library writes O = 0 and lse = -inf (a convention of this library).
 *
 * Numerics: bf16 (fp16) inputs on the matrix cores are multiplied with fp32 accumulation;
 * probabilities are rounded to bf16 (fp16) for the P V product while the normaliser (and so
 * the log-sum-exp) sums them unrounded in fp32; O is rounded to the output dtype once
 * (round to nearest even). On the general path (fp32, fp16, other widths or layouts)
 * every step is fp32 after the exact conversion of the inputs. Results equal the definition up to
 * rounding ("exact" means the same function, not the same bits). For a fixed build,
 * device, shape and input, results are bitwise reproducible from run to run: there are
 * no floating-point atomics and partial results are merged in a fixed order.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_VERSION 100 /* major * 100 + minor */

/* Status codes. Every validation happens before any device work is enqueued: a call
 * that returns an error other than FA_ERR_LAUNCH has launched nothing. Errors of the
 * asynchronous device work itself surface at the caller's next synchronisation. */
typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,      /* q, k, v or out is NULL (with B*H*N > 0), or strides NULL where needed */
  FA_ERR_SHAPE = -2,     /* negative size, size too large, or d, dv outside 1..256 */
  FA_ERR_DTYPE = -3,     /* dtype is not FA_F32, FA_BF16 or FA_F16 (gradients: not a 16-bit type) */
  FA_ERR_MASK = -4,      /* mask_mode is not FA_MASK_NONE or FA_MASK_CAUSAL */
  FA_ERR_STRIDE = -5,    /* a negative stride, rows of out / lse that overlap, or a bf16
                            k / v row stride of 2^24 elements or more */
  FA_ERR_ALIGN = -6,     /* a base pointer not aligned to its element size (bias, lse: 4 bytes) */
  FA_ERR_ALIAS = -7,     /* out or lse overlaps an input, or out overlaps lse */
  FA_ERR_WORKSPACE = -8, /* workspace NULL or smaller than fa_fwd_workspace_size() */
  FA_ERR_LAUNCH = -9,    /* the HIP runtime refused the launch */
  FA_ERR_DEVICE = -10,   /* the current HIP device is not a gfx950 */
  FA_ERR_ALLOC = -11     /* the library-owned workspace could not be allocated */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1, FA_F16 = 2 } fa_dtype;

typedef enum { FA_MASK_NONE = 0, FA_MASK_CAUSAL = 1 } fa_mask_mode;

/* Element strides (not bytes). The innermost axis of every tensor is contiguous:
 * the d axis of q and k, the dv axis of v and out, the key axis j of the bias and
 * the n axis of lse. Strides must be >= 0; 0 broadcasts (inputs only). */
typedef struct {
  int64_t q[3];    /* q[b, h, n, :] at q + b*q[0] + h*q[1] + n*q[2]          */
  int64_t k[3];    /* same for k                                             */
  int64_t v[3];    /* same for v                                             */
  int64_t out[3];  /* same for out                                           */
  int64_t bias[3]; /* bias[b, h, i, :] at bias + b*bias[0] + h*bias[1] + i*bias[2] */
  int64_t lse[2];  /* lse[b, h, :] at lse + b*lse[0] + h*lse[1]                */
} fa_strides;

/*
 * fa_fwd — attention forward, enqueued on `stream`.
 *
 * q, k:   device pointers, dtype `dtype`, logical shape [B, H, N, d].
 * v:      device pointer, dtype `dtype`, logical shape [B, H, N, dv].
 * bias:   NULL, or a device pointer to fp32 values of logical shape [B, H, N, N]
 *         (b or h stride 0 to broadcast); -inf entries forbid keys.
 * mask_mode: FA_MASK_NONE or FA_MASK_CAUSAL (added to the bias when both are given).
 * out:    device pointer, dtype `dtype`, logical shape [B, H, N, dv]; fully written.
 * lse:    NULL (not written) or a device pointer to fp32 [B, H, N]; fully written.
 * B, H, N: batch, heads, sequence length (>= 0; B*H*N == 0 returns FA_OK at once).
 * d, dv:  Q/K width and V/O width, each 1..256.
 * strides: element strides of every tensor (see fa_strides); NULL means contiguous
 *         [B, H, N, *] tensors, a contiguous [B, H, N, N] bias and a contiguous lse.
 * dtype:  FA_BF16 (bf16 q, k, v, out; fp32 accumulation), FA_F16 (the same in fp16) or
 *         FA_F32 (all fp32).
 * stream: a hipStream_t (NULL = the default stream).
 *
 * Alignment: q, k, v and out aligned to their element size; bias and lse 4-byte
 * aligned. Paths: bf16 or fp16 with d, dv in {64, 128}, 16-byte aligned q/k/v/out bases
 * and row strides, and k/v row strides below 2^24 elements runs on the matrix cores; every
 * other valid call runs on the general (vector ALU) kernel, which computes the same
 * recurrence in fp32 from the converted inputs.
 * Ownership: all pointers are caller-owned device memory; the library keeps none of
 * them after the call's device work finishes, and never mutates q, k, v or bias.
 * Scratch memory (the page "编译器与内核", section "生态系统也是目标的一部分", counts a
 * library's workspace limits, determinism and stream semantics as part of its contract):
 * split problems (few, long query tiles) need a workspace of
 * fa_fwd_workspace_size() bytes. fa_fwd takes it from one library-owned buffer per
 * (device, stream), shared with fa_bwd (calls on one stream run in order, so they
 * never use it at once; calls on different streams use different buffers). The buffer
 * only grows: a larger need allocates a new one and keeps the old one allocated until
 * fa_shutdown(), so it is safe for several host threads to call on one stream. While
 * `stream` is capturing a graph, fa_fwd returns FA_ERR_WORKSPACE for any problem that
 * needs scratch memory (a captured graph would keep reusing the shared buffer); use
 * fa_fwd_ex there. Split problems run as one kernel on `stream`: workgroups over key
 * ranges, then workgroups that merge each query tile's ranges once those have
 * published their states; under graph capture the merge is a second kernel instead.
 * Returns FA_OK or a negative fa_status (see above). Asynchronous (the page
 * "AI Infra 第5章图解: 算子与运行时", section 5.1, defines a launch as returning before
 * the device computes): the call returns before the device work finishes.
 */
int fa_fwd(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
           void* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
           const fa_strides* strides, int dtype, void* stream);

/*
 * fa_fwd_workspace_size — bytes of scratch memory that fa_fwd_ex needs for this
 * problem (0 when the problem needs none): the split partial states of the blockwise
 * method (any partition of the keys into blocks gives the same result, the page
 * "编译器与内核", section "FlashAttention 围绕 IO 改写算法"), one slot per key range of
 * (128 * dv) output values in the input dtype, 2 * 128 fp32 row statistics and an
 * 8-byte flag. Depends only on its arguments and the current device's compute-unit
 * count. Returns 0 for invalid arguments as well.
 */
size_t fa_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
                             int dtype, int mask_mode);

/*
 * fa_fwd_ex — fa_fwd with caller-provided scratch memory; allocates nothing (the
 * workspace contract of the page "编译器与内核", section "生态系统也是目标的一部分").
 * Safe under graph capture.
 * workspace: device memory of at least fa_fwd_workspace_size(...) bytes, 256-byte
 * aligned; its contents need no initialisation and are scratch after the call. It may
 * be NULL when the size is 0. Two calls that may run concurrently must not share a
 * workspace.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
              void* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
              const fa_strides* strides, int dtype, void* stream, void* workspace,
              size_t workspace_bytes);

/*
 * fa_fwd_qk — fa_fwd with N_q query rows against N_k keys (N_q, N_k >= 0). The
 * definition (the page "编译器与内核", section "FlashAttention 围绕 IO 改写算法") is
 * row-wise, so N_q rows against N_k keys are the same formula; the causal alignment
 * below is this library's reading (the pages fix none for N_q != N_k).
 * q: [B, H, N_q, d]; k: [B, H, N_k, d]; v: [B, H, N_k, dv]; out: [B, H, N_q, dv];
 * lse: NULL or [B, H, N_q]; bias: NULL or fp32 [B, H, N_q, N_k] (strides as fa_strides,
 * whose n axes are then N_q for q, out, bias rows and lse, and N_k for k and v; NULL
 * strides mean contiguous tensors of these shapes). Causal mask: key j is allowed for
 * query i iff j <= i + N_k - N_q; rows with no allowed key (N_q > N_k, or N_k = 0) get
 * O = 0, lse = -inf. k and v may be NULL when N_k = 0. Otherwise as fa_fwd (which is
 * fa_fwd_qk with N_q = N_k = N).
 */
int fa_fwd_qk(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
              void* out, float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
              int64_t dv, const fa_strides* strides, int dtype, void* stream);

/* Scratch bytes fa_fwd_qk_ex needs (0 when none, or for invalid arguments); as
 * fa_fwd_workspace_size. */
size_t fa_fwd_qk_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                int64_t dv, int dtype, int mask_mode);

/* fa_fwd_qk with caller-provided scratch memory (as fa_fwd_ex); allocates nothing and
 * is safe under graph capture. */
int fa_fwd_qk_ex(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
                 void* out, float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                 int64_t dv, const fa_strides* strides, int dtype, void* stream, void* workspace,
                 size_t workspace_bytes);

/*
 * fa_fwd_qk_noalloc — fa_fwd_qk for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc): it calls
 * no allocating routine. Split problems take their scratch memory from a fixed device
 * array of FA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each GPU it runs on
 * until the process ends (every forward plan fits: at most 512 key-range units of
 * dv <= 128); a problem whose plan needed more would return FA_ERR_WORKSPACE. All calls
 * on one GPU share that array and leave their partial states in it, so calls that may
 * overlap on one GPU (other streams, other host threads) race: serialise them, or use
 * fa_fwd_qk_ex with separate workspaces. The array needs no clearing between calls.
 * Arguments, results and other errors as fa_fwd_qk (with N_q = N_k = N it is fa_fwd).
 */
#define FA_NOALLOC_SCRATCH_BYTES 17305600
int fa_fwd_qk_noalloc(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
                      void* out, float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                      int64_t dv, const fa_strides* strides, int dtype, void* stream);

/* Static description of a status code (never NULL). Errors are part of the contract
 * surface (the page "编译器与内核", section "生成内核需要一名挑剔的评估者", item
 * 契约表面); this library reports them as status codes only. */
const char* fa_status_string(int status);

/* FA_VERSION of the loaded library (ABI compatibility is part of a library's contract:
 * the page "编译器与内核", section "生态系统也是目标的一部分"). */
int fa_version(void);

/* Frees the library-owned workspaces of fa_fwd and fa_bwd, including the retired ones
 * (synchronises each device first): the runtime's buffer lifetimes (the page
 * "编译器与内核", section "内核实现一份有边界的契约", the runtime row of its table).
 * Call it only when no call of this library is in flight and no captured graph that
 * used fa_fwd or fa_bwd will be replayed. */
void fa_shutdown(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */

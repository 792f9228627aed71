// Internal interface between the host dispatcher (fa_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Most query tiles of a plan that splits over keys (split plans have fewer query
// tiles than the GPU has compute units).
constexpr int kMaxSplitQTiles = 256;
// Most units (workgroups) of a split plan.
constexpr int kMaxSplitUnits = 512;

// Everything a forward kernel needs, passed by value as the kernel argument.
// Strides are in elements; the innermost axis of every tensor is contiguous.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const float* bias;  // nullptr: no bias
  void* out;
  float* lse;         // nullptr: lse not written
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t b_sb, b_sh, b_si;
  int64_t l_sb, l_sh;
  int B, H, N, d, dv; // N: keys (rows of K and V)
  int Nq;             // query rows (rows of Q, O, lse); N_q = N for square problems
  int coff;           // causal mask: key j allowed for query i iff j <= i + coff (= N - N_q)
  int causal;
  int bias_vec4;      // bias base 16-byte aligned and row stride a multiple of 4
  int gtile;          // general fp32 kernel: tile shape of the tile experiment (0: default)
  float scale_log2;   // log2(e) / sqrt(d): scores in base-2 units
  float scale;        // 1 / sqrt(d)
  // Work decomposition. A unit is (batch*head, query tile, range of key tiles).
  int n_qt;           // query tiles per (b, h)
  int split;          // 1: query tiles cut into key ranges (see unit_info), merged afterwards
  // Scratch for split problems: one slot per unit.
  void* part_o;      // [slot][BM/32][dv/4][32][4] normalised partial outputs (input dtype)
  float* part_ml;     // [slot][2][BM]       reference (base 2) and normaliser
  // Merge inside the forward kernel: blocks n_units .. gridDim.x-1 merge the split query
  // tiles; unit u publishes its partial state by storing `seq` (a number unique to this
  // call) into part_flag[u]. part_flag = nullptr: a separate merge kernel follows.
  uint64_t* part_flag;
  uint64_t seq;
  int n_units;        // forward units (blocks 0 .. n_units-1)
  int unit_shift;     // split plans: the unit table counts key tiles in granules of 2^unit_shift
  int merge_groups;   // merge blocks per split tile and b*h (row groups that hold query rows)
  // Split plans: the query tiles cut into more than one range, from the last one (the
  // merge blocks take them in this order; which tiles are cut depends on the cost model,
  // so they need not be the last ones). Units enumerate query tiles from the last one;
  // split tile i is query tile qt, which owns units ubase .. ubase + B*H*nch - 1, nch
  // ranges for each (b, h): split_info[i] = ubase | nch << 10 | qt << 16, so a merge
  // block finds everything about its tile in one word.
  uint32_t split_info[kMaxSplitQTiles];
  int n_split;        // split query tiles
  // Split plans: unit u is query tile (unit_info[u] & 0xff), key tiles from
  // ((>> 8) & 0x1ff) << unit_shift, count ((>> 17) & 0x1ff) << unit_shift (the last range
  // of a tile is clipped to the tile's key tiles), b*h (>> 26), so a workgroup decodes its
  // unit with one load. With a single query tile, bits 0-7 hold b*h's low 8 bits and
  // bits 26-31 its next 6 (b*h < 2^14).
  uint32_t unit_info[kMaxSplitUnits];
};

// Query-tile height of the matrix-core kernel, and the key-tile width.
constexpr int kMfmaBM = 128;
constexpr int kMfmaBN = 64;
// Most key ranges a split query tile is cut into (the merge kernel's bound).
constexpr int kMaxRanges = 16;
// Merge blocks per split query tile when each of a block's 256 threads merges `items`
// 16-byte chunks (rows of 8 * items at dv = 128, 16 * items at dv = 64).
constexpr int merge_groups(int dv, int items) { return kMfmaBM * dv / (1024 * items); }
// Items per thread of the merge blocks inside the forward kernel (fewer, larger blocks:
// they hold a forward kernel's resources) and of the separate merge kernel.
constexpr int kFusedMergeItems = 2;
// Query-tile height of the general (vector ALU) kernel.
constexpr int kGenericBM = 64;

// Gradient split plans: most units, most tiles per (b, h), most chunks per tile.
constexpr int kMaxBwdUnits = 512;
constexpr int kMaxBwdTiles = 256;
constexpr int kMaxBwdChunks = 16;

// Everything the gradient kernels need, passed by value as the kernel argument.
// Strides are in elements; the innermost axis of every tensor is contiguous.
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;    // O of the forward
  const void* dout;   // upstream gradient dO
  const float* lse;   // natural-log log-sum-exp of the forward, [B, H, N]
  const float* bias;  // nullptr: no bias
  void* grad_q;
  void* grad_k;
  void* grad_v;
  // Workspace: per (b, h) and group of 64 rows, 64 values of -lse * sqrt(d) (-inf for
  // rows past N or rows without an allowed key) then 64 values of -D_i = -dO_i . O_i.
  float* rowstat;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int64_t b_sb, b_sh, b_si;
  int64_t l_sb, l_sh;
  int B, H, N, d, dv;
  int n_grp;          // groups of 64 rows per (b, h) in rowstat: ceil(N / 128) * 2
  int causal;
  int bias_vec4;      // bias base 16-byte aligned and every bias stride a multiple of 4
  float scale_log2;   // log2(e) / sqrt(d)
  float scale;        // 1 / sqrt(d)
  float sqrt_d;
  int n_kv_blocks;    // blocks 0 .. n_kv_blocks-1 form dK, dV; the rest form dQ
  // Split plans (few tiles): a tile's steps (query steps of a key tile, key tiles of a
  // query tile) are cut into consecutive chunks, one unit each. Units of a tile with
  // more than one chunk write fp32 partial sums that a reduction kernel adds in chunk
  // order. Unit u (dK/dV units first, then dQ units) is tile (unit[u] & 0xff), steps
  // from ((>> 8) & 0x1ff), count ((>> 17) & 0x1ff), b*h (>> 26). Within a kind the
  // units run over tiles in launch order (key tiles from the first, query tiles from
  // the last under a causal mask, else from the first), then b*h, then chunks.
  int split;
  int n_tiles;        // key tiles = query tiles per (b, h)
  float* part;        // dK/dV units: [slot][128][d + dv], then dQ units: [slot][128][d]
  int64_t part_q_off; // float offset of the dQ partials
  uint32_t unit[kMaxBwdUnits];
  uint8_t nch_kv[kMaxBwdTiles], nch_q[kMaxBwdTiles];  // chunks per tile
};

// Byte i of a byte table in the kernel arguments, read through its aligned 32-bit word.
// (Indexing such tables directly let this compiler form a scalar load whose base
// address was the table base plus a byte index, shared with a 32-bit table indexed the
// same way; scalar loads drop the low two address bits, so that load read the
// neighbouring entry.)
__device__ __forceinline__ int kernarg_byte(const uint8_t* table, int i) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(table)[i >> 2];
  return (int)((w >> (8 * (i & 3))) & 0xffu);
}

// Fields of a split tile's word (Params::split_info).
__device__ __host__ __forceinline__ constexpr uint32_t split_word(int ubase, int nch, int qt) {
  return (uint32_t)ubase | (uint32_t)nch << 10 | (uint32_t)qt << 16;
}
__device__ __forceinline__ int split_ubase(uint32_t w) { return (int)(w & 0x3ffu); }
__device__ __forceinline__ int split_nch(uint32_t w) { return (int)((w >> 10) & 0x1fu); }
__device__ __forceinline__ int split_qtile(uint32_t w) { return (int)((w >> 16) & 0xffu); }

// Kernel arguments are passed by value; keep them within the 4 KiB argument block.
static_assert(sizeof(Params) <= 4096, "forward kernel arguments exceed 4 KiB");
static_assert(sizeof(BwdParams) <= 4096, "gradient kernel arguments exceed 4 KiB");

// Key rows per dK/dV workgroup and query rows per dQ workgroup of the gradient kernel.
constexpr int kBwdKT = 128;
constexpr int kBwdQT = 128;

// Launchers (each returns the hipError_t of the launch).
// grid: forward units; merge: whether split query tiles need the merge kernel.
// fp16: fp16 inputs and outputs (else bf16).
hipError_t launch_mfma(const Params& p, int grid, bool merge, bool fp16, hipStream_t stream);
// dtype: an fa_dtype value (FA_F32, FA_BF16, FA_F16).
hipError_t launch_generic(const Params& p, int dtype, hipStream_t stream);
// Gradients dQ, dK, dV (bf16, or fp16 when fp16): row statistics, one grid of `grid`
// dK/dV and dQ units, then (split plans) the reduction of the chunk partials.
hipError_t launch_bwd(const BwdParams& p, int grid, bool fp16, hipStream_t stream);

// Kernel-timestamp timing of the main kernels (fwd_mfma, fwd_generic, bwd_mfma). The timing
// probe arms pairs of events on the calling thread; each main-kernel launch on that thread
// takes the next armed pair, or none when nothing is armed (the normal case).
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
LaunchEvents next_launch_events();

}  // namespace fa

// Launches a main kernel: with an armed pair of events, through hipExtLaunchKernelGGL,
// which stamps the events with the kernel's own start and end; otherwise as usual.
#define FA_LAUNCH_MAIN(kernel, grid, block, stream, ...)                                        \
  do {                                                                                         \
    const ::fa::LaunchEvents fa_ev_ = ::fa::next_launch_events();                              \
    if (fa_ev_.start)                                                                          \
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, fa_ev_.start, fa_ev_.stop, 0u,     \
                            __VA_ARGS__);                                                      \
    else                                                                                       \
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                         \
  } while (0)

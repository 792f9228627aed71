/*
 * fa_plan.h — inspection of the work plan that fa_fwd (include/fa.h) runs, for tests
 * and tools. It needs no GPU and is not needed to call the attention forward.
 *
 * Problems whose (batch, head, query tile) triples leave compute units idle are
 * "split": each query tile's key tiles are cut into consecutive ranges (units), whose
 * partial states are merged afterwards — the blockwise form of the page "编译器与内核"
 * (Compilers and kernels), section "FlashAttention 围绕 IO 改写算法", allows any
 * partition of the keys into blocks.
 */
#ifndef FA_PLAN_H_
#define FA_PLAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t split;           /* 1: query tiles cut into key ranges, merged afterwards */
  int32_t n_qtiles;        /* query tiles per (b, h) (0 for the fp32 path) */
  int32_t qtile_rows;      /* query rows per query tile */
  int32_t key_tile;        /* keys per key tile */
  int32_t units;           /* forward workgroups */
  int32_t merge_blocks;    /* merge workgroups appended to the forward grid (split plans) */
  size_t workspace_bytes;  /* as fa_fwd_workspace_size */
  int32_t unit_tile_shift; /* unit table: first key tile and count in granules of 2^shift tiles */
} fa_plan_info;

/*
 * fa_plan_describe — the plan of a problem (arguments as for fa_fwd_workspace_size)
 * on a device with `compute_units` compute units. Writes *info (required). If the plan
 * splits and unit_info is not NULL, also writes its unit table, max_units entries at
 * most, one 32-bit word per unit in grid order: query tile (bits 0-7), first key tile
 * (8-16) and number of key tiles (17-25), both in granules of 2^info->unit_tile_shift
 * key tiles (the count rounded up; the kernel clips a tile's last range to the tile's
 * key tiles), b*h (26-31); with a single query tile, bits 0-7 hold b*h's low 8 bits and
 * bits 26-31 its next 6. Units enumerate the query tiles from the last one; a tile's
 * units are b*h-major, key ranges in order.
 * Returns FA_OK, FA_ERR_SHAPE / FA_ERR_DTYPE / FA_ERR_MASK for invalid arguments, or
 * FA_ERR_NULL when info is NULL or compute_units < 1. Thread-safe; no device calls.
 */
int fa_plan_describe(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype, int mask_mode,
                     int compute_units, fa_plan_info* info, uint32_t* unit_info, int max_units);

/* fa_plan_describe for N_q query rows against N_k keys (the plan fa_fwd_qk runs). */
int fa_plan_describe_qk(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, int dtype,
                        int mask_mode, int compute_units, fa_plan_info* info, uint32_t* unit_info,
                        int max_units);

#ifdef __cplusplus
}
#endif

#endif /* FA_PLAN_H_ */

// Gradients of the bf16 (and fp16) attention forward on the gfx950 matrix cores (MFMA),
// fp32 accumulation. (Written for bf16 below; the fp16 kernels are the same templates with
// fp16 operands, v_mfma_f32_32x32x16_f16, and fp16 P, dS and gradients.)
//
// The page "编译器与内核" (Compilers and kernels), section "FlashAttention 围绕 IO 改写算法",
// notes that the backward pass recomputes the score and probability blocks rather
// than keeping them. The gradients themselves are the chain rule of the forward
// definition S = Q K^T / sqrt(d) + C, P = rowsoftmax(S), O = P V:
//     P_ij = exp(S_ij - lse_i),            D_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),
//     dQ = dS K / sqrt(d),   dK = dS^T Q / sqrt(d).
// P is recomputed block by block from the forward's log-sum-exp, so neither the scores
// nor the probabilities ever reach memory. C gets no gradient.
//
// Mapping onto CDNA4 (this file's own design):
//  * A row-statistics kernel forms -lse_i * sqrt(d) and -D_i (D_i = dO_i . O_i) for
//    every row and stores them in groups of 64 rows (-inf for rows past N or rows with
//    no allowed key, so that their probabilities are exactly 0). They are the start
//    values of the score and dP accumulators: the matrix cores then deliver
//    sqrt(d) (S - lse) and dP - D, and P, dS cost one exponential and two multiplies.
//    (S here includes C: S - lse = Q K^T / sqrt(d) + C - lse.)
//  * One grid holds two kinds of workgroups (4 waves each). dK/dV blocks own 128 keys
//    (32 per wave) and stream the query rows in steps of 64; dQ blocks own 128 query
//    rows (32 per wave) and stream the keys in steps of 64. Every sum is formed inside
//    one workgroup in a fixed order: no atomics, bitwise reproducible.
//  * dK/dV blocks: with the wave's K and V rows held as B operands in registers,
//    S = Q K^T and dP = dO V^T come out with one key per lane (lane l: key l mod 32,
//    16 of a 32-row query block); the bf16-rounded P and dS in these registers are
//    directly the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A operands
//    (dO^T, Q^T) are transposing LDS reads (ds_read_b64_tr_b16) of the same tiles that
//    fed S and dP. lse and D of the lane's 16 rows are four 16-byte LDS reads each.
//  * dQ blocks mirror the forward: S^T = K Q^T and dP^T = V dO^T with the wave's Q and
//    dO rows held as B operands (one query per lane, so lse and D are per-lane
//    scalars), then dQ^T += K^T dS^T with K^T read transposed from the K tile.
//  * A bias enters the same start value (sqrt(d) C_ij is added to -lse_i sqrt(d)), so
//    the base-2 exponent of P is always the accumulator times log2(e)/sqrt(d).
//  * Tiles go from global memory straight into LDS (buffer loads with the LDS
//    destination), two stages, one barrier per step. Q, dO (dK/dV blocks) and K (dQ
//    blocks) are read both row-wise and transposed, so their rows use one XOR swizzle
//    of the 16-byte chunks that keeps both reads free of bank conflicts: key(row) =
//    s(row mod 4) ^ ((row / 4) mod 4), s = (0, 10, 4, 14).
//  * Few tiles (fewer dK/dV blocks than CUs): each tile's loop is cut into chunks of
//    about equal length, one workgroup each; chunks write fp32 partial sums and a
//    reduction kernel adds them in chunk order (deterministic) into the gradients.
//  * Causal: a dK/dV block starts at the query step of its first key; a dQ block ends
//    at the key tile of its last row; waves skip blocks that lie entirely in the
//    masked triangle, and element masks use the same comparison as the forward.

#include <climits>
#include <type_traits>

#include "fa_internal.h"
#include "fa_mfma_common.h"

namespace fa {
namespace {

template <int D, int DV>
struct BwdCfg {
  static constexpr int NT = 256;
  static constexpr int KT = kBwdKT;  // keys of a dK/dV block
  static constexpr int QS = 64;      // query rows per step of a dK/dV block
  static constexpr int QT = kBwdQT;  // query rows of a dQ block
  static constexpr int KS = 64;      // keys per step of a dQ block
  static constexpr int QTILE = QS * D * 2;
  static constexpr int OTILE = QS * DV * 2;
  static constexpr int VEC = 2 * QS * 4;  // lse*log2(e) and D of a query step
  static constexpr int KTILE = KS * D * 2;
  static constexpr int VTILE = KS * DV * 2;
  static constexpr int STAGE_KV = QTILE + OTILE + VEC;
  static constexpr int STAGE_Q = KTILE + VTILE;
  static constexpr int STAGE = STAGE_KV > STAGE_Q ? STAGE_KV : STAGE_Q;
};

// Chunk swizzle of tiles read both row-wise and transposed (see the header comment).
__device__ __forceinline__ constexpr int dual_key(int row) {
  return ((row & 1) * 10 + (row & 2) * 2) ^ ((row >> 2) & 3);
}

// Copy of rows r0 .. r0 + ROWS - 1 of a [N, W] bf16 matrix (row stride sn elements) into
// an LDS tile of ROWS x W, 16 bytes per lane per instruction, chunk-swizzled by
// dual_key. Lane `lane` of instruction i of wave `wave` fills the 16-byte slot
// (wave*NLD + i)*64 + lane: row slot/CH, physical chunk slot%CH, which holds logical
// chunk (slot%CH) ^ key(row). The buffer resource covers only the rows below N, so rows
// past the end read as zeros.
template <int W, int ROWS>
struct TileCopy2 {
  static constexpr int CH = W / 8;
  static constexpr int NLD = ROWS * W * 2 / (256 * 16);
  static_assert(NLD >= 1 && ROWS * W * 2 == NLD * 256 * 16, "tile must be a whole number of block copies");
  int off[NLD];
  __device__ __forceinline__ void init(int64_t sn, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int slot = (wave * NLD + i) * 64 + lane;
      const int row = slot / CH;
      off[i] = (int)(row * sn * 2) + ((slot % CH) ^ (dual_key(row) & (CH - 1))) * 16;
    }
  }
  // r: the buffer resource of the tile's rows (rows_rsrc)
  __device__ __forceinline__ void copy(unsigned char* dst, __amdgpu_buffer_rsrc_t r, int wave) const {
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, dst + (wave * NLD + i) * 1024), 16, off[i], 0, 0, 0);
  }
};

// Buffer resource over rows r0 .. r0 + ROWS - 1 of a matrix (row stride sn elements) that
// covers only the rows below N.
template <int ROWS, typename E>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const E* base, int64_t sn, int r0, int N) {
  const int rows = min(ROWS, N - r0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(base + (int64_t)r0 * sn), 0, rows * (int)sn * 2,
                                           kBufferWord3);
}

// Operand reads from a dual-swizzled LDS tile of W bf16 per row. A read's byte offset
// within the tile is a per-lane base XOR a compile-time constant (the swizzled chunk
// index is an XOR, and the fields it touches are disjoint from the row's), so one
// register per kind of read serves every k-step and column block.
template <typename E, int W>
struct TileReads {
  typedef typename Vec<E>::v8 e8;
  typedef typename Vec<E>::v4 e4;
  static constexpr int CH = W / 8;
  int rbase;     // row-wise read: row l32 (+32*blk), logical chunk 2*kk + g -> rbase ^ 32*kk
  int tbase[2];  // transposing read, half hh: column block db -> tbase[hh] ^ 64*db
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, l32 = lane & 31;
    // (2kk + g) ^ key = 2kk ^ (g ^ key): offset (l32*W*2 | 16 (g ^ key)) ^ 32 kk
    rbase = (l32 * (W * 2)) | (((g ^ dual_key(l32)) & (CH - 1)) * 16);
    // Transposing read (A operand with k = 16 rows of group sg): within a 16-lane group
    // G, lane L reads row 16*sg + 8*hh + 4*g + L/4 at columns c0 .. c0+3,
    // c0 = 32*db + c1, c1 = 16*(G&1) + 4*(L&3); the row's swizzle key does not depend
    // on sg, and (4*db + c1/8) ^ key = 4*db ^ (c1/8 ^ key).
    const int G = lane >> 4, L = lane & 15;
    const int c1 = 16 * (G & 1) + 4 * (L & 3);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = 8 * hh + 4 * g + (L >> 2);
      const int key = dual_key(row) & (CH - 1);
      tbase[hh] = (row * (W * 2)) | ((((c1 >> 3) ^ key) & (CH - 1)) * 16) | ((c1 & 7) * 2);
    }
  }
  // A or B operand: row 32*blk + (lane mod 32), k = 16*kk + 8*g .. +7
  __device__ __forceinline__ e8 row(const unsigned char* t, int blk, int kk) const {
    return *reinterpret_cast<const e8*>(t + blk * 32 * (W * 2) + (rbase ^ (32 * kk)));
  }
  // A operand of a product over the tile's rows: column 32*db + (lane mod 32), with k
  // running over the 16 rows of group sg in the order the accumulator layout holds them.
  __device__ __forceinline__ e8 tr(const unsigned char* t, int sg, int db) const {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        LDS_PTR(i16x4, t + 16 * sg * (W * 2) + (tbase[0] ^ (64 * db))));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        LDS_PTR(i16x4, t + 16 * sg * (W * 2) + (tbase[1] ^ (64 * db))));
    e8 a;
    a.lo = __builtin_bit_cast(e4, lo);
    a.hi = __builtin_bit_cast(e4, hi);
    return a;
  }
};

// Row statistics: 16 threads per row. rowstat group layout: see BwdParams.
template <typename E, int DV>
__global__ __launch_bounds__(256) void bwd_rowstat(BwdParams p) {
  constexpr int EL = DV / 16;  // elements per thread
  const int row = blockIdx.x * 16 + threadIdx.x / 16;
  const int part = threadIdx.x % 16;
  const int Np = p.n_grp * 64;
  const int bh = row / Np, i = row % Np;
  const int b = bh / p.H, h = bh % p.H;
  float acc = 0.f;
  // the row's lse is loaded with O and dO (one memory round trip, not two)
  const float lse = part == 0 && i < p.N ? p.lse[b * p.l_sb + h * p.l_sh + i] : 0.f;
  if (i < p.N) {
    const E* o = static_cast<const E*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_sn + part * EL;
    const E* g = static_cast<const E*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)i * p.do_sn + part * EL;
    typedef E vec_t __attribute__((ext_vector_type(EL)));
    const vec_t ov = *reinterpret_cast<const vec_t*>(o);
    const vec_t gv = *reinterpret_cast<const vec_t*>(g);
#pragma unroll
    for (int e = 0; e < EL; ++e) acc = fmaf((float)ov[e], (float)gv[e], acc);
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (part == 0) {
    // -lse * sqrt(d): the start value of a score accumulator, so that it ends holding
    // sqrt(d) * (S_ij - lse_i) without C; -inf where no probability may arise
    float m = -INFINITY;
    if (i < p.N) m = lse == -INFINITY ? -INFINITY : -lse * p.sqrt_d;
    float* grp = p.rowstat + ((int64_t)bh * p.n_grp + i / 64) * 128;
    grp[i % 64] = m;
    grp[64 + i % 64] = i < p.N ? -acc : 0.f;  // -D: the start value of a dP accumulator
  }
}

// One unit of the gradient grid: tile `tile` of b*h `bh`, steps [s_begin, s_end) of its
// loop; `partial`: the tile is cut into several chunks, so the unit writes fp32
// partial sums into its slot instead of the bf16 gradient.
struct BwdUnit {
  int bh, tile, s_begin, s_end, slot;
  bool partial;
};

// query steps (of QS = 64 rows) of key tile kt, from the first one its keys can see
__device__ __forceinline__ int kv_steps(const BwdParams& p, int kt) {
  const int qs0 = p.causal ? kt * kBwdKT : 0;
  return (p.N - qs0 + 63) / 64;
}
// key tiles (of 64 keys) of query tile qt
__device__ __forceinline__ int q_steps(const BwdParams& p, int qt) {
  const int nt = (p.N + 63) / 64;
  return p.causal ? min(nt, (qt * kBwdQT + kBwdQT - 1) / 64 + 1) : nt;
}

// Unit u of a kind (dK/dV or dQ units, numbered from 0 within the kind). Without a split
// the units are (tile, b*h) pairs, longest tiles first; with one they come from the table.
__device__ __forceinline__ BwdUnit bwd_unit(const BwdParams& p, int u, bool kv) {
  const int BH = p.B * p.H;
  BwdUnit w;
  w.slot = u;
  if (!p.split) {
    w.bh = u % BH;
    const int r = u / BH;
    w.tile = kv || !p.causal ? r : p.n_tiles - 1 - r;
    w.s_begin = 0;
    w.s_end = kv ? kv_steps(p, w.tile) : q_steps(p, w.tile);
    w.partial = false;
    return w;
  }
  const unsigned info = p.unit[(kv ? u : p.n_kv_blocks + u) % kMaxBwdUnits];
  w.tile = (int)(info & 0xff);
  w.s_begin = (int)((info >> 8) & 0x1ff);
  w.s_end = w.s_begin + (int)((info >> 17) & 0x1ff);
  w.bh = (int)(info >> 26);
  w.partial = kernarg_byte(kv ? p.nch_kv : p.nch_q, w.tile) > 1;
  return w;
}

// ---- dK, dV of 128 keys of one (b, h) ----
template <typename E, int D, int DV, bool BIAS>
__device__ void dkdv_block(const BwdParams& p, int blk, unsigned char* st0, unsigned char* st1) {
  using C = BwdCfg<D, DV>;
  typedef typename Vec<E>::v8 e8;
  typedef typename Vec<E>::v4 e4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const BwdUnit U = bwd_unit(p, blk, true);
  const int bh = U.bh, kt = U.tile;
  const int b = bh / p.H, h = bh % p.H;
  const int N = p.N;
  const int k0 = kt * C::KT;
  const int wk0 = k0 + wave * 32;
  const int key = wk0 + l32;  // this lane's key
  const bool kvalid = key < N;

  const E* qp = static_cast<const E*>(p.q) + b * p.q_sb + h * p.q_sh;
  const E* gp = static_cast<const E*>(p.dout) + b * p.do_sb + h * p.do_sh;
  const E* kp = static_cast<const E*>(p.k) + b * p.k_sb + h * p.k_sh;
  const E* vp = static_cast<const E*>(p.v) + b * p.v_sb + h * p.v_sh;
  const float* stat = p.rowstat + (int64_t)bh * p.n_grp * 128;

  // K^T and V^T as B operands: lane holds its key, dims 16*kk + 8*g .. +7
  e8 kreg[D / 16], vreg[DV / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    kreg[kk] = kvalid ? *reinterpret_cast<const e8*>(kp + (int64_t)key * p.k_sn + kk * 16 + g * 8) : e8{};
#pragma unroll
  for (int kk = 0; kk < DV / 16; ++kk)
    vreg[kk] = kvalid ? *reinterpret_cast<const e8*>(vp + (int64_t)key * p.v_sn + kk * 16 + g * 8) : e8{};

  const float* bcol = nullptr;  // bias column of this lane's key (rows added per element)
  if constexpr (BIAS) bcol = p.bias + b * p.b_sb + h * p.b_sh + min(key, N - 1);

  TileCopy2<D, C::QS> qcp;
  TileCopy2<DV, C::QS> gcp;
  qcp.init(p.q_sn, wave, lane);
  gcp.init(p.do_sn, wave, lane);
  TileReads<E, D> qr;
  TileReads<E, DV> gr;
  qr.init(lane);
  gr.init(lane);

  // query steps: causal blocks start at the step that holds their first key; this
  // unit runs steps U.s_begin .. U.s_end - 1 of them
  const int qs0 = (p.causal ? (k0 / C::QS) * C::QS : 0) + U.s_begin * C::QS;
  const int nsteps = U.s_end - U.s_begin;
  auto copy_step = [&](unsigned char* st, int qs) {
    qcp.copy(st, rows_rsrc<C::QS>(qp, p.q_sn, qs, N), wave);
    gcp.copy(st + C::QTILE, rows_rsrc<C::QS>(gp, p.do_sn, qs, N), wave);
    if (wave == 0 && lane < 32) {  // the step's 64 lse and 64 D values: one 512-byte group
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(stat + (qs / 64) * 128), 0, 512, kBufferWord3);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, st + C::QTILE + C::OTILE), 16, lane * 16, 0, 0, 0);
    }
  };

  floatx16 dkacc[D / 32], dvacc[DV / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dkacc[i] = floatx16{};
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) dvacc[i] = floatx16{};

  if (nsteps > 0) copy_step(st0, qs0);
  for (int s = 0; s < nsteps; ++s) {
    unsigned char* cur = (s & 1) ? st1 : st0;
    unsigned char* nxt = (s & 1) ? st0 : st1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // step s has landed; every wave is done with step s-1's stage
    const int qs = qs0 + s * C::QS;
    if (s + 1 < nsteps) copy_step(nxt, qs + C::QS);
    const unsigned char* qt_ = cur;
    const unsigned char* gt_ = cur + C::QTILE;
    const float* vec = reinterpret_cast<const float*>(cur + C::QTILE + C::OTILE);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qb0 = qs + qb * 32;
      if (p.causal && qb0 + 31 < wk0) continue;  // every (row, key) of the block is masked
      if (qb0 >= N) continue;
      // The accumulators start from the rows' statistics (register r holds row
      // qb0 + 8*(r/4) + 4*g + r%4): S from sqrt(d) (C - lse), dP from -D.
      floatx16 sacc, dpacc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const floatx4 m4 = *reinterpret_cast<const floatx4*>(vec + qb * 32 + 8 * j + 4 * g);
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(vec + 64 + qb * 32 + 8 * j + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sacc[4 * j + e] = m4[e];
          dpacc[4 * j + e] = d4[e];
        }
      }
      if constexpr (BIAS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb0 + 8 * (r >> 2) + 4 * g + (r & 3);
          sacc[r] = fmaf(bcol[(int64_t)min(q, N - 1) * p.b_si], p.sqrt_d, sacc[r]);
        }
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) sacc = mfma32(qr.row(qt_, qb, kk), kreg[kk], sacc);
#pragma unroll
      for (int kk = 0; kk < DV / 16; ++kk) dpacc = mfma32(gr.row(gt_, qb, kk), vreg[kk], dpacc);
      e8 pk[2], dsk[2];
      // P and dS of the block. Causal mask: key > row, i.e. kd > 8*(r/4) + r%4 with
      // kd = key - qb0 - 4g; it never fires on blocks below the diagonal, and kd is made
      // the smallest int without a causal mask.
      const int kd = p.causal ? key - qb0 - 4 * g : INT_MIN;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // base-2 exponent of P: sqrt(d) (S - lse) * log2(e) / sqrt(d)
        float pr = __builtin_amdgcn_exp2f(sacc[r] * p.scale_log2);
        pr = kd > 8 * (r >> 2) + (r & 3) ? 0.f : pr;
        pk[r >> 3][r & 7] = (E)pr;
        dsk[r >> 3][r & 7] = (E)(pr * dpacc[r]);
      }
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) dvacc[db] = mfma32(gr.tr(gt_, 2 * qb + kq, db), pk[kq], dvacc[db]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) dkacc[db] = mfma32(qr.tr(qt_, 2 * qb + kq, db), dsk[kq], dkacc[db]);
      }
    }
  }

  if (!kvalid) return;
  // accumulator register r of block db holds column key, dim 32*db + 8*(r/4) + 4*g + r%4
  if (U.partial) {  // raw sums into the unit's slot: [128 keys][d + dv] fp32
    float* pp = p.part + ((int64_t)U.slot * C::KT + (key - k0)) * (D + DV);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<floatx4*>(pp + db * 32 + r4 * 8 + g * 4) =
            floatx4{dkacc[db][r4 * 4], dkacc[db][r4 * 4 + 1], dkacc[db][r4 * 4 + 2], dkacc[db][r4 * 4 + 3]};
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<floatx4*>(pp + D + db * 32 + r4 * 8 + g * 4) =
            floatx4{dvacc[db][r4 * 4], dvacc[db][r4 * 4 + 1], dvacc[db][r4 * 4 + 2], dvacc[db][r4 * 4 + 3]};
    return;
  }
  E* dkp = static_cast<E*>(p.grad_k) + b * p.dk_sb + h * p.dk_sh + (int64_t)key * p.dk_sn;
  E* dvp = static_cast<E*>(p.grad_v) + b * p.dv_sb + h * p.dv_sh + (int64_t)key * p.dv_sn;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      e4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)(dkacc[db][r4 * 4 + e] * p.scale);
      *reinterpret_cast<e4*>(dkp + db * 32 + r4 * 8 + g * 4) = o4;
    }
#pragma unroll
  for (int db = 0; db < DV / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      e4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)dvacc[db][r4 * 4 + e];
      *reinterpret_cast<e4*>(dvp + db * 32 + r4 * 8 + g * 4) = o4;
    }
}

// ---- dQ of 128 query rows of one (b, h) ----
template <typename E, int D, int DV, bool BIAS>
__device__ void dq_block(const BwdParams& p, int blk, unsigned char* st0, unsigned char* st1) {
  using C = BwdCfg<D, DV>;
  typedef typename Vec<E>::v8 e8;
  typedef typename Vec<E>::v4 e4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const BwdUnit U = bwd_unit(p, blk, false);
  const int bh = U.bh, qt = U.tile;
  const int b = bh / p.H, h = bh % p.H;
  const int N = p.N;
  const int wq0 = qt * C::QT + wave * 32;
  const int qi = wq0 + l32;  // this lane's query row
  const bool qvalid = qi < N;

  const E* qp = static_cast<const E*>(p.q) + b * p.q_sb + h * p.q_sh;
  const E* gp = static_cast<const E*>(p.dout) + b * p.do_sb + h * p.do_sh;
  const E* kp = static_cast<const E*>(p.k) + b * p.k_sb + h * p.k_sh;
  const E* vp = static_cast<const E*>(p.v) + b * p.v_sb + h * p.v_sh;

  // Q^T and dO^T as B operands: lane holds its row, dims 16*kk + 8*g .. +7
  e8 qreg[D / 16], greg[DV / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qreg[kk] = qvalid ? *reinterpret_cast<const e8*>(qp + (int64_t)qi * p.q_sn + kk * 16 + g * 8) : e8{};
#pragma unroll
  for (int kk = 0; kk < DV / 16; ++kk)
    greg[kk] = qvalid ? *reinterpret_cast<const e8*>(gp + (int64_t)qi * p.do_sn + kk * 16 + g * 8) : e8{};
  const int qc = min(qi, N - 1);
  const float* grp = p.rowstat + ((int64_t)bh * p.n_grp + qc / 64) * 128;
  // base-2 exponent of P: (sqrt(d) (Q K^T/sqrt(d) + C) - lse sqrt(d)) log2(e)/sqrt(d)
  const float mcs = qvalid ? grp[qc % 64] * p.scale_log2 : -INFINITY;  // -lse log2(e)
  const float ndrow = qvalid ? grp[64 + qc % 64] : 0.f;                 // -D
  const float* brow = nullptr;
  if constexpr (BIAS) brow = p.bias + b * p.b_sb + h * p.b_sh + (int64_t)qc * p.b_si;

  TileCopy2<D, C::KS> kcp;
  TileCopy2<DV, C::KS> vcp;
  kcp.init(p.k_sn, wave, lane);
  vcp.init(p.v_sn, wave, lane);
  TileReads<E, D> kr;
  TileReads<E, DV> vr;
  kr.init(lane);
  vr.init(lane);

  // key tiles U.s_begin .. U.s_end - 1; a wave skips those above its own rows
  const int t_begin = U.s_begin, t_end = U.s_end;
  const int tw_end = p.causal ? min(t_end, (wq0 + 31) / C::KS + 1) : t_end;
  auto copy_step = [&](unsigned char* st, int t) {
    kcp.copy(st, rows_rsrc<C::KS>(kp, p.k_sn, t * C::KS, N), wave);
    vcp.copy(st + C::KTILE, rows_rsrc<C::KS>(vp, p.v_sn, t * C::KS, N), wave);
  };

  floatx16 dqacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dqacc[i] = floatx16{};

  if (t_begin < t_end) copy_step(st0, t_begin);
  for (int t = t_begin; t < t_end; ++t) {
    unsigned char* cur = ((t - t_begin) & 1) ? st1 : st0;
    unsigned char* nxt = ((t - t_begin) & 1) ? st0 : st1;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // tile t has landed; every wave is done with tile t-1's stage
    if (t + 1 < t_end) copy_step(nxt, t + 1);
    if (t >= tw_end) continue;
    const unsigned char* kt_ = cur;
    const unsigned char* vt_ = cur + C::KTILE;
    const int kv0 = t * C::KS;
    // The row's lse and D are per-lane scalars here, so the accumulators start from 0
    // (sqrt(d) C with a bias) and the statistics enter in the element loop; start
    // values that are the same in every register would hold 32 registers for the loop.
    floatx16 sacc[2], dpacc[2];
    const bool bvec = BIAS && p.bias_vec4 && kv0 + C::KS <= N;  // 4 keys per 16-byte load
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[kb][r] = 0.f;
        dpacc[kb][r] = 0.f;
      }
      if constexpr (BIAS) {
        // register r holds key kv0 + 32 kb + 8 (r/4) + 4 g + r%4
        if (bvec) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const floatx4 b4 = *reinterpret_cast<const floatx4*>(brow + kv0 + kb * 32 + 8 * r4 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[kb][4 * r4 + e] = b4[e] * p.sqrt_d;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][r] = brow[min(kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3), N - 1)] * p.sqrt_d;
        }
      }
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) sacc[kb] = mfma32(kr.row(kt_, kb, kk), qreg[kk], sacc[kb]);
#pragma unroll
      for (int kk = 0; kk < DV / 16; ++kk) dpacc[kb] = mfma32(vr.row(vt_, kb, kk), greg[kk], dpacc[kb]);
    }
    e8 dsk[4];
    // dS of the tile; tiles that cross the diagonal or the sequence end mask keys
    auto dscores = [&](auto MASKc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float ds_even = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], p.scale_log2, mcs));
          if constexpr (decltype(MASKc)::value) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key >= N || (p.causal && key > qi)) pr = 0.f;
          }
          const float ds = pr * (dpacc[kb][r] + ndrow);
          if (r & 1)  // elements r - 1 and r as one packed word
            set_pair(dsk[kb * 2 + (r >> 3)], (r & 7) >> 1, cvt_pk<E>(ds_even, ds));
          else
            ds_even = ds;
        }
      }
    };
    if (kv0 + C::KS > N || (p.causal && kv0 + C::KS - 1 > wq0))
      dscores(std::true_type{});
    else
      dscores(std::false_type{});
#pragma unroll
    for (int sg = 0; sg < 4; ++sg)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) dqacc[db] = mfma32(kr.tr(kt_, sg, db), dsk[sg], dqacc[db]);
  }

  if (!qvalid) return;
  if (U.partial) {  // raw sums into the unit's slot: [128 rows][d] fp32
    float* pp = p.part + p.part_q_off + ((int64_t)U.slot * C::QT + (qi - qt * C::QT)) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<floatx4*>(pp + db * 32 + r4 * 8 + g * 4) =
            floatx4{dqacc[db][r4 * 4], dqacc[db][r4 * 4 + 1], dqacc[db][r4 * 4 + 2], dqacc[db][r4 * 4 + 3]};
    return;
  }
  E* dqp = static_cast<E*>(p.grad_q) + b * p.dq_sb + h * p.dq_sh + (int64_t)qi * p.dq_sn;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      e4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)(dqacc[db][r4 * 4 + e] * p.scale);
      *reinterpret_cast<e4*>(dqp + db * 32 + r4 * 8 + g * 4) = o4;
    }
}

template <typename E, int D, int DV, bool BIAS>
__global__ __launch_bounds__(256, 2) void bwd_mfma(BwdParams p) {
  using C = BwdCfg<D, DV>;
  __shared__ __attribute__((aligned(16))) unsigned char st0[C::STAGE], st1[C::STAGE];
  if ((int)blockIdx.x < p.n_kv_blocks)
    dkdv_block<E, D, DV, BIAS>(p, blockIdx.x, st0, st1);
  else
    dq_block<E, D, DV, BIAS>(p, blockIdx.x - p.n_kv_blocks, st0, st1);
}

// Sum of the chunk partials of split tiles, in chunk order, into the bf16 gradients.
// Block (row group of kReduceRows, b*h, tile): tile < n_tiles is a key tile (dK, dV),
// else a query tile (dQ). Tiles with a single chunk were written by their unit. Small
// row groups give each thread one or two items, whose chunk loads are all in flight
// together.
constexpr int kReduceRows = 8;
template <typename E, int D, int DV>
__global__ __launch_bounds__(256) void bwd_reduce(BwdParams p) {
  typedef typename Vec<E>::v4 e4;
  const int bh = blockIdx.y;
  const bool kv = (int)blockIdx.z < p.n_tiles;
  const int tile = kv ? blockIdx.z : blockIdx.z - p.n_tiles;
  const int nch = kernarg_byte(kv ? p.nch_kv : p.nch_q, tile);
  if (nch <= 1) return;
  const int b = bh / p.H, h = bh % p.H;
  const int W = kv ? D + DV : D;  // floats per row of a slot
  // first slot of the tile: the units of the tiles launched before it, then b*h
  const uint8_t* nch_of = kv ? p.nch_kv : p.nch_q;
  const bool rev = !kv && p.causal;
  int before = 0;
  for (int t = rev ? p.n_tiles - 1 : 0; t != tile; t += rev ? -1 : 1) before += kernarg_byte(nch_of, t);
  const int slot0 = before * p.B * p.H + bh * nch;
  const float* base = p.part + (kv ? 0 : p.part_q_off) + (int64_t)slot0 * 128 * W;
  const int n4 = kReduceRows * W / 4;  // float4 items of the block's rows
  for (int it = threadIdx.x; it < n4; it += 256) {
    const int r = blockIdx.x * kReduceRows + it / (W / 4);  // row within the tile
    const int c = (it % (W / 4)) * 4;              // column within the slot row
    // every chunk's load is issued before the sum (fixed order j = 0, 1, ...)
    floatx4 v[kMaxBwdChunks];
#pragma unroll
    for (int j = 0; j < kMaxBwdChunks; ++j)
      if (j < nch) v[j] = *reinterpret_cast<const floatx4*>(base + ((int64_t)j * 128 + r) * W + c);
    floatx4 acc = v[0];
#pragma unroll
    for (int j = 1; j < kMaxBwdChunks; ++j)
      if (j < nch) acc += v[j];
    const int n = tile * 128 + r;
    if (n >= p.N) continue;
    e4 o4;
    E* dst;
    if (kv && c >= D) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)acc[e];
      dst = static_cast<E*>(p.grad_v) + b * p.dv_sb + h * p.dv_sh + (int64_t)n * p.dv_sn + (c - D);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)(acc[e] * p.scale);
      dst = kv ? static_cast<E*>(p.grad_k) + b * p.dk_sb + h * p.dk_sh + (int64_t)n * p.dk_sn + c
               : static_cast<E*>(p.grad_q) + b * p.dq_sb + h * p.dq_sh + (int64_t)n * p.dq_sn + c;
    }
    *reinterpret_cast<e4*>(dst) = o4;
  }
}

#define FA_BWD_VARIANTS(E)                                      \
  template __global__ void bwd_mfma<E, 64, 64, false>(BwdParams);   \
  template __global__ void bwd_mfma<E, 64, 64, true>(BwdParams);    \
  template __global__ void bwd_mfma<E, 64, 128, false>(BwdParams);  \
  template __global__ void bwd_mfma<E, 64, 128, true>(BwdParams);   \
  template __global__ void bwd_mfma<E, 128, 64, false>(BwdParams);  \
  template __global__ void bwd_mfma<E, 128, 64, true>(BwdParams);   \
  template __global__ void bwd_mfma<E, 128, 128, false>(BwdParams); \
  template __global__ void bwd_mfma<E, 128, 128, true>(BwdParams);  \
  template __global__ void bwd_rowstat<E, 64>(BwdParams);           \
  template __global__ void bwd_rowstat<E, 128>(BwdParams);          \
  template __global__ void bwd_reduce<E, 64, 64>(BwdParams);        \
  template __global__ void bwd_reduce<E, 64, 128>(BwdParams);       \
  template __global__ void bwd_reduce<E, 128, 64>(BwdParams);       \
  template __global__ void bwd_reduce<E, 128, 128>(BwdParams);
FA_BWD_VARIANTS(__bf16)
FA_BWD_VARIANTS(_Float16)
#undef FA_BWD_VARIANTS

template <typename E, int D, int DV>
hipError_t launch_bwd_dd(const BwdParams& p, int grid, hipStream_t stream) {
  const int rows = p.B * p.H * p.n_grp * 64;
  hipLaunchKernelGGL((bwd_rowstat<E, DV>), dim3(rows / 16), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.bias)
    FA_LAUNCH_MAIN((bwd_mfma<E, D, DV, true>), dim3(grid), dim3(256), stream, p);
  else
    FA_LAUNCH_MAIN((bwd_mfma<E, D, DV, false>), dim3(grid), dim3(256), stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || !p.split) return e;
  hipLaunchKernelGGL((bwd_reduce<E, D, DV>), dim3(kBwdKT / kReduceRows, p.B * p.H, 2 * p.n_tiles), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_bwd_e(const BwdParams& p, int grid, hipStream_t stream) {
  if (p.d == 128 && p.dv == 128) return launch_bwd_dd<E, 128, 128>(p, grid, stream);
  if (p.d == 64 && p.dv == 128) return launch_bwd_dd<E, 64, 128>(p, grid, stream);
  if (p.d == 128 && p.dv == 64) return launch_bwd_dd<E, 128, 64>(p, grid, stream);
  if (p.d == 64 && p.dv == 64) return launch_bwd_dd<E, 64, 64>(p, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int grid, bool fp16, hipStream_t stream) {
  return fp16 ? launch_bwd_e<_Float16>(p, grid, stream) : launch_bwd_e<__bf16>(p, grid, stream);
}

}  // namespace fa

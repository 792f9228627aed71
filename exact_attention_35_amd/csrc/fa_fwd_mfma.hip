// bf16 attention forward on the gfx950 matrix cores (MFMA), fp32 accumulation.
//
// Method: the online-softmax recurrence of the page "编译器与内核" (Compilers and
// kernels), section "FlashAttention 围绕 IO 改写算法": a workgroup keeps a tile of
// query rows on chip, streams key/value blocks through LDS, and for each block forms
// the scores, the block max b_t, the running max m_t, alpha_t = exp(m_{t-1} - m_t),
// the normaliser l_t and the numerator o_t, writing O_i = o_T / l_T at the end. The
// N x N scores and probabilities exist only in registers.
//
// Mapping onto CDNA4 (all of it is this file's own design):
//  * A workgroup is 4 waves and owns BM = 128 query rows; wave w owns 32 rows. A key
//    tile is BN = 64 keys.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (A = 32 keys x 16 dims from LDS, B = 16 dims x 32 queries held in VGPRs for the
//    whole kernel). In the 32x32 accumulator, lane l holds query (l mod 32) and 16 of
//    the block's 32 keys; lane l^32 holds the other 16. So the row max and row sum
//    are per-lane reductions plus one exchange between the two half-waves.
//  * The same accumulator registers, rounded to bf16, are directly the B operand of
//    O^T = V^T P^T (A = 32 dv x 16 keys from LDS). For that, the V tile is stored
//    transposed in LDS (one row per dv) with its 64 key positions permuted (bits 2
//    and 3 of the key index swapped) so that the 8 keys a lane needs for one MFMA
//    are contiguous: one 16-byte LDS read per operand.
//  * The O^T accumulator again has one query per lane, so the rescale by alpha_t is a
//    per-lane scalar multiply.
//  * Exponentials in base 2 (v_exp_f32): scores are carried as S*log2(e); the factor
//    is folded into the 1/sqrt(d) scale. Probabilities are rounded to bf16 once
//    (v_cvt_pk_bf16_f32, round to nearest even) and the normaliser sums the rounded
//    values, so O is a convex combination of V rows.
//  * K rows and transposed V rows are padded by 16 bytes in LDS so that the 16-byte
//    operand reads of 8 consecutive lanes hit distinct banks.
//  * K/V tiles are double-buffered: the global loads of tile t+1 are issued into
//    registers before tile t is computed and written to the other LDS stage after.
//  * Causal: key tiles entirely above a query tile's diagonal are never visited; a
//    wave whose 32 rows all precede a key tile skips it; element masks are applied
//    only on tiles that cross the diagonal or the sequence end.
//  * Split over keys (for problems with too few query tiles to fill 256 CUs): a
//    query tile's key tiles are cut into n_split contiguous ranges (the recurrence
//    allows any partition of the keys into blocks). Each range writes its partial
//    state (o, m, l) to scratch memory, takes an arrival ticket, and the last range to
//    arrive merges all partials in fixed range order — deterministic, no atomics on
//    data. The merge of two partial states over disjoint key sets is
//    m = max(m_a, m_b), l = 2^(m_a-m) l_a + 2^(m_b-m) l_b, o likewise.

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, int DV>
struct Cfg {
  static constexpr int NWAVES = 4;
  static constexpr int NT = NWAVES * 64;
  static constexpr int BM = kMfmaBM;            // 128 = NWAVES * 32
  static constexpr int BN = kMfmaBN;            // 64
  static constexpr int KROW = D * 2 + 16;       // bytes per K row in LDS
  static constexpr int VROW = BN * 2 + 16;      // bytes per transposed V row (one dv)
  static constexpr int KTILE = BN * KROW;
  static constexpr int VTILE = DV * VROW;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int KK = D / 16;             // MFMA k-steps of Q K^T
  static constexpr int NDB = DV / 32;           // 32-wide dv blocks of P V
  static constexpr int KCH = D / 8;             // 16-byte chunks per K row
  static constexpr int KLOADS = BN * KCH / NT;  // K chunks per thread per tile
  static constexpr int VPAIRS = 16 * (DV / 8);  // (4-key group, 8-dv chunk) pairs
  static constexpr int VLOADS = (VPAIRS + NT - 1) / NT;
  static_assert(BM == NWAVES * 32, "one 32-row block per wave");
  static_assert(BN * KCH % NT == 0, "K tile loader shape");
};

// LDS position of key k (0..63) inside a transposed V row: bits 2 and 3 swapped.
__device__ __forceinline__ int vpos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int DV>
struct TileRegs {
  u32x4 k[Cfg<D, DV>::KLOADS];
  u32x4 v[Cfg<D, DV>::VLOADS][4];
};

// Global -> registers for key tile starting at kv0 (rows >= N read as zero).
template <int D, int DV>
__device__ __forceinline__ void load_tile(TileRegs<D, DV>& r, const __bf16* kp, const __bf16* vp,
                                          int64_t k_sn, int64_t v_sn, int kv0, int N, int tid) {
  using C = Cfg<D, DV>;
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int id = i * C::NT + tid;
    const int row = id / C::KCH, ch = id % C::KCH;
    const int key = kv0 + row;
    r.k[i] = key < N ? *reinterpret_cast<const u32x4*>(kp + (int64_t)key * k_sn + ch * 8) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < C::VLOADS; ++i) {
    const int id = i * C::NT + tid;
    if (id < C::VPAIRS) {
      const int c = id / 16, j = id % 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = kv0 + 4 * j + u;
        r.v[i][u] = key < N ? *reinterpret_cast<const u32x4*>(vp + (int64_t)key * v_sn + c * 8)
                            : u32x4{0, 0, 0, 0};
      }
    }
  }
}

// Registers -> LDS stage (K row-major, V transposed with permuted key positions).
template <int D, int DV>
__device__ __forceinline__ void store_tile(const TileRegs<D, DV>& r, unsigned char* stage, int tid) {
  using C = Cfg<D, DV>;
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int id = i * C::NT + tid;
    const int row = id / C::KCH, ch = id % C::KCH;
    *reinterpret_cast<u32x4*>(stage + row * C::KROW + ch * 16) = r.k[i];
  }
  unsigned char* vt = stage + C::KTILE;
#pragma unroll
  for (int i = 0; i < C::VLOADS; ++i) {
    const int id = i * C::NT + tid;
    if (id < C::VPAIRS) {
      const int c = id / 16, j = id % 16;
      const int pos = vpos(4 * j);
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // dword w of each key row = dv pair (2w, 2w+1)
        const uint32_t a0 = r.v[i][0][w], a1 = r.v[i][1][w], a2 = r.v[i][2][w], a3 = r.v[i][3][w];
        u32x2 lo, hi;
        lo[0] = (a0 & 0xffffu) | (a1 << 16);
        lo[1] = (a2 & 0xffffu) | (a3 << 16);
        hi[0] = (a0 >> 16) | (a1 & 0xffff0000u);
        hi[1] = (a2 >> 16) | (a3 & 0xffff0000u);
        const int dv = c * 8 + 2 * w;
        *reinterpret_cast<u32x2*>(vt + dv * C::VROW + pos * 2) = lo;
        *reinterpret_cast<u32x2*>(vt + (dv + 1) * C::VROW + pos * 2) = hi;
      }
    }
  }
}

template <int D, int DV>
__global__ __launch_bounds__(256, 2) void fwd_mfma(Params p) {
  using C = Cfg<D, DV>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[C::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;    // half-wave
  const int l32 = lane & 31;  // query within the wave's 32-row block

  // ---- work unit: (b*h, query tile, key split); causal tiles longest first ----
  const int u = blockIdx.x;
  const int sp = u % p.n_split;
  const int rr = u / p.n_split;
  const int BH = p.B * p.H;
  const int bh = rr % BH;
  const int qt = p.causal ? (p.n_qt - 1 - rr / BH) : (rr / BH);
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int q0 = qt * C::BM;
  const int kv_len = p.causal ? min(p.N, q0 + C::BM) : p.N;
  const int ntiles = (kv_len + C::BN - 1) / C::BN;
  const int t_begin = (int)((int64_t)sp * ntiles / p.n_split);
  const int t_end = (int)((int64_t)(sp + 1) * ntiles / p.n_split);
  if (t_begin >= t_end) return;  // empty range (only when ntiles < n_split)

  const __bf16* qp = static_cast<const __bf16*>(p.q) + b * p.q_sb + h * p.q_sh;
  const __bf16* kp = static_cast<const __bf16*>(p.k) + b * p.k_sb + h * p.k_sh;
  const __bf16* vp = static_cast<const __bf16*>(p.v) + b * p.v_sb + h * p.v_sh;

  // ---- Q^T operand: lane holds query (wq0 + l32), dims kk*16 + g*8 .. +8 ----
  const int wq0 = q0 + wave * 32;
  const int qi = wq0 + l32;
  const bool qvalid = qi < p.N;
  bf16x8 qreg[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
    if (qvalid) {
      qreg[kk] = *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.q_sn + kk * 16 + g * 8);
    } else {
      qreg[kk] = bf16x8{};
    }
  }
  const float* brow = (p.bias && qvalid) ? p.bias + b * p.b_sb + h * p.b_sh + (int64_t)qi * p.b_si : nullptr;

  floatx16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = floatx16{};
  float m_run = -INFINITY;  // running max (base 2), same in both half-waves
  float l_run = 0.f;        // this half-wave's share of the running normaliser

  TileRegs<D, DV> regs;
  load_tile<D, DV>(regs, kp, vp, p.k_sn, p.v_sn, t_begin * C::BN, p.N, tid);
  store_tile<D, DV>(regs, smem, tid);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int kv0 = t * C::BN;
    const int s = (t - t_begin) & 1;
    const bool has_next = t + 1 < t_end;
    if (has_next) load_tile<D, DV>(regs, kp, vp, p.k_sn, p.v_sn, kv0 + C::BN, p.N, tid);

    const unsigned char* ks = smem + s * C::STAGE;
    const unsigned char* vt = ks + C::KTILE;
    const bool wave_active = !(p.causal && kv0 > wq0 + 31);
    if (wave_active) {
      // ---- S^T = K Q^T for keys kv0 .. kv0+63 (two 32-key blocks) ----
      floatx16 sacc[2] = {floatx16{}, floatx16{}};
#pragma unroll
      for (int kk = 0; kk < C::KK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + l32) * C::KROW + kk * 32 + g * 16);
          sacc[kb] = mfma32(a, qreg[kk], sacc[kb]);
        }
      }
      // ---- scale, bias, mask: x = S*log2e/sqrt(d) + C*log2e ----
      // register r of block kb holds key kv0 + kb*32 + (r/4)*8 + g*4 + r%4
      const bool edge = (kv0 + C::BN > p.N) || (p.causal && kv0 + C::BN - 1 > wq0);
      float bmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int key0 = kv0 + kb * 32 + r4 * 8 + g * 4;
          float bv[4] = {0.f, 0.f, 0.f, 0.f};
          if (brow) {
            if (p.bias_vec4 && key0 + 3 < p.N) {
              const floatx4 t4 = *reinterpret_cast<const floatx4*>(brow + key0);
              bv[0] = t4[0]; bv[1] = t4[1]; bv[2] = t4[2]; bv[3] = t4[3];
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) bv[e] = key0 + e < p.N ? brow[key0 + e] : 0.f;
            }
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = sacc[kb][r4 * 4 + e] * p.scale_log2;
            if (brow) x = fmaf(bv[e], kLog2e, x);
            if (edge) {
              const int key = key0 + e;
              if (key >= p.N || (p.causal && key > qi)) x = -INFINITY;
            }
            sacc[kb][r4 * 4 + e] = x;
            bmax = fmaxf(bmax, x);
          }
        }
      }
      // ---- block max b_t, running max m_t, alpha_t ----
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const float m_new = fmaxf(m_run, bmax);
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;  // no allowed key yet: add nothing
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
      m_run = m_new;
      // ---- P~ = exp2(x - m_t), rounded to bf16; l_t = alpha l + sum(P~) ----
      bf16x8 pk[2][2];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const __bf16 pb = (__bf16)__builtin_amdgcn_exp2f(sacc[kb][hs * 8 + e] - m_ref);
            pk[kb][hs][e] = pb;
            psum += (float)pb;
          }
        }
      }
      l_run = alpha * l_run + psum;
      // ---- o_t = alpha o_{t-1} + P~ V  (as O^T = V^T P^T) ----
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {  // 16-key groups of the tile
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (db * 32 + l32) * C::VROW + sg * 32 + g * 16);
          oacc[db] = mfma32(a, pk[sg >> 1][sg & 1], oacc[db]);
        }
      }
    }

    if (has_next) store_tile<D, DV>(regs, smem + (s ^ 1) * C::STAGE, tid);
    __syncthreads();
  }

  // ---- epilogue ----
  // register r of dv block db holds dv = db*32 + (r/4)*8 + g*4 + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int row = wave * 32 + l32;  // row within the query tile

  if (p.n_split == 1) {
    if (!qvalid) return;
    __bf16* op = static_cast<__bf16*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)qi * p.o_sn;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][r4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + db * 32 + r4 * 8 + g * 4) = o4;
      }
    }
    if (p.lse && g == 0) {
      p.lse[b * p.l_sb + h * p.l_sh + qi] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }

  // ---- split: write this range's partial state ----
  // partial o layout per unit: [chunk c4 = dv/4][row][4] so that stores and the
  // merge's loads are contiguous across lanes.
  const int tile_id = bh * p.n_qt + qt;
  const int64_t unit = (int64_t)tile_id * p.n_split + sp;
  float* po = p.part_o + unit * (C::BM * DV);
  float* pml = p.part_ml + unit * (2 * C::BM);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c4 = db * 8 + r4 * 2 + g;
      floatx4 v4 = {oacc[db][r4 * 4 + 0], oacc[db][r4 * 4 + 1], oacc[db][r4 * 4 + 2], oacc[db][r4 * 4 + 3]};
      *reinterpret_cast<floatx4*>(po + (c4 * C::BM + row) * 4) = v4;
    }
  }
  if (g == 0) {
    pml[row] = m_run;
    pml[C::BM + row] = l_tot;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    const int nonempty = min(p.n_split, ntiles);
    const unsigned prev = __hip_atomic_fetch_add(p.counters + tile_id, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (unsigned)(nonempty - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

  // ---- last arrival: merge all partials of this query tile in range order ----
  float* wts = reinterpret_cast<float*>(smem);  // [n_split][BM] merge weights
  const float* ml0 = p.part_ml + (int64_t)tile_id * p.n_split * (2 * C::BM);
  for (int r = tid; r < C::BM; r += C::NT) {
    float m = -INFINITY;
    for (int j = 0; j < p.n_split; ++j) {
      const bool ne = (int)((int64_t)j * ntiles / p.n_split) < (int)((int64_t)(j + 1) * ntiles / p.n_split);
      if (ne) m = fmaxf(m, ml0[j * 2 * C::BM + r]);
    }
    float l = 0.f;
    if (m != -INFINITY) {
      for (int j = 0; j < p.n_split; ++j) {
        const bool ne = (int)((int64_t)j * ntiles / p.n_split) < (int)((int64_t)(j + 1) * ntiles / p.n_split);
        if (ne) l += __builtin_amdgcn_exp2f(ml0[j * 2 * C::BM + r] - m) * ml0[j * 2 * C::BM + C::BM + r];
      }
    }
    const bool ok = (m != -INFINITY) && l > 0.f;
    const float inv = ok ? 1.f / l : 0.f;
    for (int j = 0; j < p.n_split; ++j) {
      const bool ne = (int)((int64_t)j * ntiles / p.n_split) < (int)((int64_t)(j + 1) * ntiles / p.n_split);
      wts[j * C::BM + r] = (ok && ne) ? __builtin_amdgcn_exp2f(ml0[j * 2 * C::BM + r] - m) * inv : 0.f;
    }
    const int qr = q0 + r;
    if (p.lse && qr < p.N)
      p.lse[b * p.l_sb + h * p.l_sh + qr] = ok ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  }
  __syncthreads();
  const float* po0 = p.part_o + (int64_t)tile_id * p.n_split * (C::BM * DV);
  __bf16* ob = static_cast<__bf16*>(p.out) + b * p.o_sb + h * p.o_sh;
  for (int idx = tid; idx < C::BM * (DV / 4); idx += C::NT) {
    const int c4 = idx / C::BM, r = idx % C::BM;
    const int qr = q0 + r;
    if (qr >= p.N) continue;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < p.n_split; ++j) {
      const float w = wts[j * C::BM + r];
      if (w != 0.f) {
        const floatx4 v4 = *reinterpret_cast<const floatx4*>(po0 + (int64_t)j * (C::BM * DV) + (c4 * C::BM + r) * 4);
        acc += w * v4;
      }
    }
    // chunk c4 = db*8 + r4*2 + g covers dv = db*32 + r4*8 + g*4 .. +4
    const int dv0 = (c4 >> 3) * 32 + ((c4 >> 1) & 3) * 8 + (c4 & 1) * 4;
    bf16x4 o4;
#pragma unroll
    for (int e = 0; e < 4; ++e) o4[e] = (__bf16)acc[e];
    *reinterpret_cast<bf16x4*>(ob + (int64_t)qr * p.o_sn + dv0) = o4;
  }
  if (tid == 0) __hip_atomic_store(p.counters + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_mfma_bf16(const Params& p, int grid, hipStream_t stream) {
  const dim3 g(grid), blk(256);
  if (p.d == 128 && p.dv == 128) hipLaunchKernelGGL((fwd_mfma<128, 128>), g, blk, 0, stream, p);
  else if (p.d == 64 && p.dv == 128) hipLaunchKernelGGL((fwd_mfma<64, 128>), g, blk, 0, stream, p);
  else if (p.d == 128 && p.dv == 64) hipLaunchKernelGGL((fwd_mfma<128, 64>), g, blk, 0, stream, p);
  else if (p.d == 64 && p.dv == 64) hipLaunchKernelGGL((fwd_mfma<64, 64>), g, blk, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace fa

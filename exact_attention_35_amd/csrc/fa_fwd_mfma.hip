// bf16 and fp16 attention forward on the gfx950 matrix cores (MFMA), fp32 accumulation.
// (Written for bf16 below; the fp16 kernels are the same template with fp16 operands,
// v_mfma_f32_32x32x16_f16, fp16 probabilities and fp16 partial outputs.)
//
// Method: the online-softmax recurrence of the page "编译器与内核" (Compilers and
// kernels), section "FlashAttention 围绕 IO 改写算法": a workgroup keeps a tile of
// query rows on chip, streams key/value blocks through LDS, and for each block forms
// the scores, the block max b_t, the reference m_t, the rescale alpha_t, the
// normaliser l_t and the numerator o_t, writing O_i = o_T / l_T at the end. The
// N x N scores and probabilities exist only in registers.
//
// Mapping onto CDNA4 (all of it is this file's own design):
//  * A workgroup is 4 waves and owns BM = 128 query rows; wave w owns 32 rows. A key
//    tile is BN = 64 keys. Two workgroups fit on a CU (64 KiB of LDS each).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//    (A = 32 keys x 16 dims from LDS, B = 16 dims x 32 queries held in VGPRs for the
//    whole kernel). In the 32x32 accumulator, lane l holds query (l mod 32) and 16 of
//    the block's 32 keys; lane l^32 holds the other 16. Row max and row sum are
//    per-lane reductions plus one exchange between the two half-waves.
//  * The same accumulator registers, rounded to bf16, are directly the B operand of
//    O^T = V^T P^T (A = 32 dv x 16 keys). V stays row-major in LDS; the A operand is
//    read with ds_read_b64_tr_b16, which hands each lane four consecutive keys of one
//    dv column; two such reads give the 8 keys the P^T operand holds in that lane.
//  * The O^T accumulator again has one query per lane, so rescaling is a per-lane
//    scalar multiply.
//  * K and V tiles go from global memory straight into LDS (buffer_load_dwordx4 with
//    the LDS destination, no staging registers). Rows are stored with their 16-byte
//    chunks XOR-swizzled by the row index, so the operand reads of neighbouring lanes
//    hit distinct banks; the swizzle is applied on the global side of the copy. The
//    buffer resource covers only the rows that exist, so rows past the sequence end
//    read as zeros; their keys are masked in the scores.
//  * Software pipeline, one barrier per key tile: iteration t computes the scores of
//    tile t+1 (Q K^T) and the P V product of tile t-1 on the matrix cores while the
//    vector ALUs run the softmax of tile t; the copies of K(t+2) and V(t) are in flight
//    meanwhile (two LDS stages each for K and V). The body is one compile-time
//    sequence of slots (a matrix instruction, an operand read ahead, a share of the
//    softmax), with the wave's issue priority raised for its Q K^T half.
//  * Exponentials in base 2 (v_exp_f32): scores are carried as S*log2(e); the factor
//    is folded into the 1/sqrt(d) scale and into the exp argument's FMA.
//  * Lazy reference: the recurrence is exact for any reference value that bounds the
//    exponents; this kernel moves a row's reference m_t only when the block max
//    exceeds it by more than 8 (a factor 2^8), so most tiles need no rescale of o and
//    l (alpha_t = 1). Probabilities are then <= 2^8, far from fp32/bf16 limits.
//    The normaliser sums the fp32 probabilities; the bf16-rounded copies feed P V.
//  * Causal: key tiles entirely above a query tile's diagonal are never visited; a
//    wave skips the tiles that lie entirely above its own 32 rows; element masks are
//    applied only on tiles that cross the diagonal or the sequence end.
//  * Split over keys (problems with too few query tiles to fill the CUs): a query
//    tile's key tiles are cut into contiguous ranges of about equal cost (the
//    recurrence allows any partition of the keys into blocks). Each range writes its
//    partial state (its own normalised output o/l in bf16, m and l in fp32) to
//    scratch memory and publishes it; merge blocks at the end of the same grid combine
//    the ranges of each tile in range order (deterministic; no atomics):
//    m = max_p m_p, l = sum_p 2^(m_p-m) l_p, O = sum_p (2^(m_p-m) l_p / l) (o_p/l_p).

#include <type_traits>

#include "fa_internal.h"
#include "fa_mfma_common.h"

namespace fa {
namespace {

// Cache policy of a buffer store (sc0 | sc1): system scope, so the L2 writes the data
// through instead of keeping it dirty. The split partial states are read by other
// workgroups (merge blocks of the same kernel, on any XCD, or a following merge
// kernel): written through, they have reached memory once the stores complete, and the
// L2 needs no write-back of them at the kernel's end.
constexpr int kStoreWriteThrough = 1 | 16;

constexpr float kTau = 8.0f;  // lazy-reference slack, log2 units

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector-memory operations
// are outstanding and leaves the export and LDS/scalar counters unconstrained.
constexpr int vmcnt_wait(int n) { return (n & 0xf) | ((n >> 4) & 0x3) << 14 | 0x7 << 4 | 0xf << 8; }

template <int D, int DV>
struct Cfg {
  static constexpr int NT = 256;
  static constexpr int BM = kMfmaBM;   // 128
  static constexpr int BN = kMfmaBN;   // 64
  static constexpr int KCH = D / 8;    // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;   // 16-byte chunks per V row
  static constexpr int KTILE = BN * D * 2;
  static constexpr int VTILE = BN * DV * 2;
  static constexpr int LDS = 2 * KTILE + 2 * VTILE;
  static constexpr int KK = D / 16;    // MFMA k-steps of Q K^T
  static constexpr int NDB = DV / 32;  // 32-wide dv blocks of P V
  static constexpr int KLD = KTILE / (NT * 16);  // direct loads per thread per K tile
  static constexpr int VLD = VTILE / (NT * 16);
};

// Tile copies: rows kv0 .. kv0+BN-1 of a [N, W] bf16 matrix with row stride `sn`
// go into an LDS stage, 16 bytes per lane per instruction, chunk-swizzled. Lane
// `lane` of instruction i of wave `wave` fills 16-byte slot (wave*NLD + i)*64 + lane,
// i.e. row slot/CH, physical chunk slot%CH, which holds logical chunk
// (slot%CH) ^ (row mod CH). The loads go through a buffer resource whose base is the
// tile's first row and whose size covers only the rows that exist, so the per-lane
// byte offsets do not depend on the tile, and the rows past the sequence end (tail
// tile only) read as zeros instead of touching memory.
template <typename E>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const E* base, int64_t sn, int kv0, int N) {
  const int rows = min(kMfmaBN, N - kv0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(base + (int64_t)kv0 * sn), 0,
                                           rows * (int)sn * 2, kBufferWord3);
}

// XOR keys of the two LDS layouts (16-byte chunk index ^= key(row)):
//  * K rows: key = row mod CH. The A-operand read of Q K^T has 8 (or 16) lanes
//    on consecutive rows at one logical chunk, which the key spreads over distinct
//    banks.
//  * V rows: key = s(row mod 4) mod CH with s = (0, 10, 4, 14). A transposing read of
//    P V has each 16-lane group on 4 consecutive rows x 2 logical chunks, and each
//    32-lane half on 4 rows x 4 chunks; s makes both sets hit distinct banks whether
//    the LDS serves 128 or 256 bytes per clock. The key only depends on row mod 4.
__device__ __forceinline__ constexpr int v_swizzle_key(int row) { return ((row & 1) * 10 + (row & 2) * 2); }

template <int W, int NLD, bool VKEY>
struct TileCopy {
  static constexpr int CH = W / 8;
  int off[NLD];  // byte offset of this lane's 16 bytes from the tile's first row
  __device__ __forceinline__ void init(int64_t sn, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int slot = (wave * NLD + i) * 64 + lane;
      const int row = slot / CH;
      const int key = (VKEY ? v_swizzle_key(row) : row) & (CH - 1);
      off[i] = (int)(row * sn * 2) + ((slot % CH) ^ key) * 16;
    }
  }
  __device__ __forceinline__ void copy(unsigned char* stage, __amdgpu_buffer_rsrc_t r, int wave) const {
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, stage + (wave * NLD + i) * 1024), 16, off[i], 0, 0, 0);
  }
};

// Per-unit description: which (b*h, query tile) and which range of key tiles.
// `partial`: the range is one of several of its query tile, so the unit writes a
// partial state to be merged; otherwise it writes the output rows itself.
struct Unit {
  int bh, qt, t_begin, t_end, slot;
  bool partial;
};

__device__ __forceinline__ int qtile_ntiles(const Params& p, int qt, int BM, int BN) {
  const int kv_len = p.causal ? min(p.N, (qt + 1) * BM + p.coff) : p.N;
  return (max(kv_len, 0) + BN - 1) / BN;
}

// Units of a plan without a split are (b*h, query tile) pairs, longest query tile
// first; a split plan reads its unit from the table. The decode is branch-free, so the
// table entry and the plan type are read from the kernel arguments in one round trip.
// With a single query tile (decoding) the query-tile bits hold the low 8 bits of b*h.
__device__ __forceinline__ Unit decode_unit(const Params& p, int u, int BM, int BN) {
  static_assert((kMaxSplitUnits & (kMaxSplitUnits - 1)) == 0, "unit table size must be a power of two");
  const unsigned info = p.unit_info[u & (kMaxSplitUnits - 1)];  // inside the table for any plan
  const bool split = p.split != 0;
  const unsigned BH = (unsigned)(p.B * p.H);
  const unsigned r = (unsigned)u / BH;
  Unit w;
  const bool one = p.n_qt == 1;
  w.qt = split ? (one ? 0 : (int)(info & 0xff)) : (p.causal ? p.n_qt - 1 - (int)r : (int)r);
  w.bh = split ? (int)(one ? (info & 0xff) | (info >> 26) << 8 : info >> 26) : (int)((unsigned)u - r * BH);
  const int nt = qtile_ntiles(p, w.qt, BM, BN);
  // first key tile and count in granules of 2^unit_shift tiles; the last range of a
  // tile is clipped to the tile's key tiles
  w.t_begin = split ? (int)((info >> 8) & 0x1ff) << p.unit_shift : 0;
  w.t_end = split ? min(w.t_begin + ((int)((info >> 17) & 0x1ff) << p.unit_shift), nt) : nt;
  w.partial = w.t_end - w.t_begin < nt;
  w.slot = u;
  return w;
}

// ---- compile-time helpers of the interleaved tile body ----
// The softmax of one tile as a list of micro-steps, in dependency order:
//   [0, NPRE)            bias only: x = s / sqrt(d) + bias, one element each
//   MSK                  edge tiles only: causal / sequence-end element mask
//   [MAX0, MAX0 + 16)    block max: two chains of 8 steps (one chain per key block)
//   XCH                  half-wave exchange of the max, reference, alpha, -reference
//   [ELT0, ELT0+32+LAG)  step k: exponential of element k (k < 32), and the fp32 sum
//                        and bf16 conversion of element k - LAG (k >= LAG)
//   UPD                  normaliser update
// Each step has an estimated cost in clocks. The steps are spread over the first 85% of
// the NS slots of the fused tile body so that the cumulative cost grows in proportion
// (leaving the end of the Q K^T half, where the wave's priority is raised, mostly to the
// matrix cores; measured ~1% faster than spreading over all slots), except that a step
// is pulled earlier when it has a deadline: the score registers of key block 0
// (elements 0..15) are overwritten by the next tile's Q K^T from slot NP on, those of
// block 1 from slot P2 on, so every step that reads them must come before.
template <bool BIAS, bool EDGE = false, int LAG_ = 2>
struct SmPlan {
  static constexpr int LAG = LAG_;  // steps between an exponential and the use of its result
  static constexpr int NPRE = BIAS ? 32 : 0;
  static constexpr int MSK = NPRE;
  static constexpr int MAX0 = NPRE + (EDGE ? 1 : 0);
  static constexpr int XCH = MAX0 + 16;
  static constexpr int ELT0 = XCH + 1;
  static constexpr int UPD = ELT0 + 32 + LAG;
  static constexpr int NOPS = UPD + 1;
  static constexpr int cost(int k) {
    return k < NPRE ? 4 : k < MAX0 ? 96 : k < XCH ? 4 : k == XCH ? 48 : k < UPD ? 20 : 8;
  }
  static constexpr int total() {
    int c = 0;
    for (int k = 0; k < NOPS; ++k) c += cost(k);
    return c;
  }
  static constexpr int deadline(int k, int NP, int P2, int NS) {
    return k < ELT0 + 16 ? NP - 1 : k < ELT0 + 32 ? P2 - 1 : NS - 1;
  }
  // number of steps placed in slots 0 .. i-1
  static constexpr int first(int i, int NP, int P2, int NS) {
    int k = 0, c = 0;
    const int NSE = NS * 85 / 100;  // slots that share the softmax
    for (int sl = 0; sl < i; ++sl) {
      const long target = sl + 1 >= NSE ? (long)total() : (long)total() * (sl + 1) / NSE;
      while (k < NOPS && (c + cost(k) <= target || deadline(k, NP, P2, NS) <= sl)) {
        c += cost(k);
        ++k;
      }
    }
    return k;
  }
};

// Softmax state of one tile, shared by its micro-steps.
struct SmState {
  float mx[2];   // block max of the two key blocks (per lane)
  float nref;    // minus the reference, or 0 while no allowed key has been seen
  float ps[4];   // partial fp32 sums of the probabilities
  float pf[32];  // probabilities awaiting their sum and bf16 conversion
};

// ---- merge of the partial states of split query tiles ----
// One block merges RG = IT * RG1 rows of one query tile of one b*h: thread = (chunk of
// 4 dv values, IT rows RG1 apart), so the merge costs one memory round trip: every thread
// first issues the loads of its items in every range, while the first RG threads load
// their row's (m_p, l_p), turn them into weights 2^(m_p - m) l_p / l (m = max_p m_p,
// l = sum_p 2^(m_p - m) l_p) and stage them in LDS; then O = sum_p w_p (o_p / l_p) in
// range order (deterministic, and the same arithmetic for any IT), o_p / l_p being the
// normalised output each range stored.
// COHERENT: the partial states were written by workgroups of the same kernel, maybe on
// another XCD, so they are read with agent-scope loads (sc1), which do not use lines of
// the workspace that this XCD's L2 may still hold from an earlier call.
// ok = false (the ranges never published their states) makes the block's rows NaN.
constexpr int kLoadAgentScope = 16;  // buffer load cache policy: sc1

// The merge items of one thread (IT chunks of 4 dv values, rows RG1 apart) in every
// range of a split query tile, and the (m_p, l_p) of row rg*RG + tid for tid < RG.
// Ranges j >= nch keep o = 0, m = -inf, l = 0, so they weigh nothing.
template <typename E, int DV, int IT>
struct MergeItems {
  typedef typename Vec<E>::v4 e4;
  static constexpr int BM = kMfmaBM;
  static constexpr int NC4 = DV / 4;     // chunks of 4 values in a row of o
  static constexpr int RG1 = 256 / NC4;  // rows of one item per thread: 8 (dv = 128) or 16 (dv = 64)
  static constexpr int RG = IT * RG1;    // rows per block
  static_assert(BM / RG == merge_groups(DV, IT), "merge grid and block shape disagree");
  __amdgpu_buffer_rsrc_t ro, rml;
  int rg;
  int off[IT];                 // byte offset of item k within a range's slot
  u32x2 raw[IT][kMaxRanges];   // o_p / l_p, 4 bf16 values per item
  float mp[kMaxRanges], lp[kMaxRanges];

  __device__ __forceinline__ void init(const Params& p, int ubase, int bh, int rg_, int nch) {
    rg = rg_;
    const int slot0 = ubase + bh * nch;
    // slot j holds [BM/32][dv/4][32][4] bf16: row r, chunk c4 at ((r/32)*NC4 + c4)*32 + r%32
    ro = __builtin_amdgcn_make_buffer_rsrc(static_cast<E*>(p.part_o) + (int64_t)slot0 * (BM * DV), 0, nch * BM * DV * 2, kBufferWord3);
    rml = __builtin_amdgcn_make_buffer_rsrc(p.part_ml + (int64_t)slot0 * (2 * BM), 0, nch * 2 * BM * 4, kBufferWord3);
    const int rr = threadIdx.x % RG1, c4 = threadIdx.x / RG1;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int r = rg * RG + k * RG1 + rr;  // row within the query tile
      off[k] = (((r >> 5) * NC4 + c4) * 32 + (r & 31)) * 8;
    }
#pragma unroll
    for (int j = 0; j < kMaxRanges; ++j) {
#pragma unroll
      for (int k = 0; k < IT; ++k) raw[k][j] = u32x2{0u, 0u};
      mp[j] = -INFINITY;
      lp[j] = 0.f;
    }
  }
  // issues the loads of range J (cache policy POL)
  template <int J, int POL>
  __device__ __forceinline__ void load() {
#pragma unroll
    for (int k = 0; k < IT; ++k) raw[k][J] = __builtin_amdgcn_raw_buffer_load_b64(ro, off[k] + J * (BM * DV * 2), 0, POL);
    if ((int)threadIdx.x < RG) {
      const int r = rg * RG + threadIdx.x;
      mp[J] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rml, (J * 2 * BM + r) * 4, 0, POL));
      lp[J] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rml, (J * 2 * BM + BM + r) * 4, 0, POL));
    }
  }
  // Weights 2^(m_p - m) l_p / l (m = max_p m_p, l = sum_p 2^(m_p - m) l_p) staged in LDS by
  // the first RG threads, then O = sum_p w_p (o_p / l_p) in range order (deterministic)
  // and lse. ok = false (the ranges never published their states) makes the rows NaN.
  __device__ __forceinline__ void combine(const Params& p, int qt, int bh, float* w_s, bool ok) {
    const int b = bh / p.H, h = bh % p.H;
    const int tid = threadIdx.x;
    if (tid < RG) {
      const int qr = qt * BM + rg * RG + tid;
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < kMaxRanges; ++j) m = fmaxf(m, mp[j]);
      float w[kMaxRanges], l = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxRanges; ++j) {
        w[j] = m != -INFINITY ? __builtin_amdgcn_exp2f(mp[j] - m) : 0.f;  // 0 for absent ranges
        l += w[j] * lp[j];
      }
      const bool any = m != -INFINITY && l > 0.f;
      const float inv = !ok ? __builtin_nanf("") : any ? 1.f / l : 0.f;
#pragma unroll
      for (int j = 0; j < kMaxRanges; ++j) w_s[j * RG + tid] = ok && !any ? 0.f : w[j] * lp[j] * inv;
      if (p.lse && qr < p.Nq)
        p.lse[b * p.l_sb + h * p.l_sh + qr] =
            !ok ? __builtin_nanf("") : any ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    }
    __syncthreads();
    const int rr = tid % RG1, c4 = tid / RG1;
    // chunk c4 = db*8 + r4*2 + g covers dv = db*32 + r4*8 + g*4 .. +4
    const int dv0 = (c4 >> 3) * 32 + ((c4 >> 1) & 3) * 8 + (c4 & 1) * 4;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int qr = qt * BM + rg * RG + k * RG1 + rr;
      if (qr >= p.Nq) continue;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < kMaxRanges; ++j) {
        const e4 hv = __builtin_bit_cast(e4, raw[k][j]);
        acc += w_s[j * RG + k * RG1 + rr] * floatx4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
      }
      e4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (E)acc[e];
      E* orow = static_cast<E*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)qr * p.o_sn;
      *reinterpret_cast<e4*>(orow + dv0) = o4;
    }
  }
};

// Merge blocks of the forward kernel itself (blocks n_units on): the split query tiles
// (p.split_info, from the last one), then b*h, then groups of rows. The units of the tile
// publish their partial states by storing this call's number into their flags once the states are
// written through to memory; wave 0 polls the flags (one lane per range) with
// agent-scope loads until all of them hold it. The merge blocks come after every unit
// in the grid, so a waiting merge block never holds back a unit. The polls are bounded:
// a tile whose ranges never publish gets NaN rows instead of a hang.
constexpr int kMaxMergePolls = 1 << 20;

template <typename E, int DV>
__device__ void merge_block(const Params& p, int m, float* w_s) {
  using MI = MergeItems<E, DV, kFusedMergeItems>;
  const int groups = p.merge_groups;  // groups of rows that hold query rows (<= the tile's)
  const int BH = p.B * p.H;
  const int rg = m % groups;
  const int t = m / groups;
  const int bh = t % BH;
  const uint32_t info = p.split_info[(t / BH) % kMaxSplitQTiles];
  const int qt = split_qtile(info), nch = split_nch(info), ubase = split_ubase(info);
  const uint64_t* flag = p.part_flag + ubase + bh * nch;
  int* ready_s = reinterpret_cast<int*>(w_s + kMaxRanges * MI::RG);
  MI items;
  items.init(p, ubase, bh, rg, nch);
  // Each range's loads are issued as soon as its flag holds this call's number, so a
  // block that waits for the last ranges already holds the others.
  const unsigned all = (1u << nch) - 1u;
  unsigned loaded = 0;
  for (int it = 0; it < kMaxMergePolls && loaded != all; ++it) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const bool mine = lane < nch && __hip_atomic_load(flag + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == p.seq;
      const uint64_t ready = __builtin_amdgcn_ballot_w64(mine);
      if (lane == 0) *ready_s = (int)(unsigned)ready;
    }
    __syncthreads();
    const unsigned fresh = (unsigned)__builtin_amdgcn_readfirstlane(*ready_s) & ~loaded;
    __syncthreads();  // every wave has read the mask before wave 0 writes the next one
    static_for<0, kMaxRanges>([&](auto J) {
      if (fresh >> decltype(J)::value & 1u) items.template load<decltype(J)::value, kLoadAgentScope>();
    });
    loaded |= fresh;
    if (loaded != all) __builtin_amdgcn_s_sleep(8);
  }
  items.combine(p, qt, bh, w_s, loaded == all);
}

// Separate merge kernel (used where the forward kernel runs without merge blocks):
// block = (group of rows, b*h, split query tile) = (blockIdx.x, .y, .z).
template <typename E, int DV>
__global__ __launch_bounds__(256) void merge_split(Params p) {
  using MI = MergeItems<E, DV, 1>;
  __shared__ float w_s[kMaxRanges * MI::RG];
  const uint32_t info = p.split_info[blockIdx.z];
  // the argument cache lines used below and the tile's table entry in one round trip
  asm volatile("" ::"s"(p.out), "s"(p.o_sn), "s"(p.Nq), "s"(p.part_ml), "s"(info));
  const int qt = split_qtile(info), nch = split_nch(info);
  MI items;
  items.init(p, split_ubase(info), blockIdx.y, blockIdx.x, nch);
  static_for<0, kMaxRanges>([&](auto J) {
    if (decltype(J)::value < nch) items.template load<decltype(J)::value, 0>();
  });
  items.combine(p, qt, blockIdx.y, w_s, true);
}

template <typename E, int D, int DV, bool BIAS>
__global__ __launch_bounds__(256, 2) void fwd_mfma(Params p) {
  using C = Cfg<D, DV>;
  typedef typename Vec<E>::v8 e8;
  typedef typename Vec<E>::v4 e4;
  // LDS stages, one array each: the compiler can then tell that a copy into one stage
  // never overlaps operand reads from the other, and does not wait for the copy.
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[C::KTILE], k_lds1[C::KTILE];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[C::VTILE], v_lds1[C::VTILE];

  // One word of each cache line of the kernel arguments that the prologue reads, and the
  // unit's table entry, are read before anything depends on them (before the branch to
  // the merge blocks too): these scalar loads share one memory round trip, and later
  // argument reads hit the scalar cache (a dependent chain of argument reads costs a
  // round trip per cache line).
  asm volatile("" ::"s"(p.q), "s"(p.k_sn), "s"(p.b_si), "s"(p.split), "s"(p.n_units),
               "s"(p.unit_info[blockIdx.x & (kMaxSplitUnits - 1)]));
  if ((int)blockIdx.x >= p.n_units) {  // merge block (the LDS stages are free for it)
    merge_block<E, DV>(p, blockIdx.x - p.n_units, reinterpret_cast<float*>(k_lds0));
    return;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;    // half-wave
  const int l32 = lane & 31;  // query within the wave's 32-row block

  const Unit U = decode_unit(p, blockIdx.x, C::BM, C::BN);
  const int b = U.bh / p.H;
  const int h = U.bh % p.H;
  const int q0 = U.qt * C::BM;
  const int N = p.N;

  const E* qp = static_cast<const E*>(p.q) + b * p.q_sb + h * p.q_sh;
  const E* kp = static_cast<const E*>(p.k) + b * p.k_sb + h * p.k_sh;
  const E* vp = static_cast<const E*>(p.v) + b * p.v_sb + h * p.v_sh;

  // ---- Q^T operand: lane holds query (wq0 + l32), dims kk*16 + g*8 .. +8 ----
  const int wq0 = q0 + wave * 32;
  const int qi = wq0 + l32;
  const bool qvalid = qi < p.Nq;
  const int qlim = qi + p.coff;  // causal: this row's last allowed key
  e8 qreg[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
    qreg[kk] = qvalid ? *reinterpret_cast<const e8*>(qp + (int64_t)qi * p.q_sn + kk * 16 + g * 8) : e8{};

  // bias row of this lane's query (rows past N read row N-1; their results are dropped)
  const float* brow = nullptr;
  if constexpr (BIAS) brow = p.bias + b * p.b_sb + h * p.b_sh + (int64_t)min(qi, p.Nq - 1) * p.b_si;

  // tiles this wave computes: causal tiles entirely above its rows are skipped, and a
  // wave whose rows all lie past the last query row computes nothing
  const int t_begin = U.t_begin, t_end = U.t_end;
  const int wlast = wq0 + 31 + p.coff;  // causal: last key the wave's last row may see
  const int tw_end = wq0 >= p.Nq ? t_begin
                     : p.causal  ? (wlast < 0 ? t_begin : min(t_end, wlast / C::BN + 1))
                                 : t_end;

  // ---- per-lane operand addresses (bytes within a stage) ----
  // K operand: row kb*32 + l32, logical chunk 2*kk + g, physical chunk
  // (2*kk + g) ^ (row mod KCH); row mod KCH does not depend on kb (KCH divides 32), so
  // kb only adds an immediate offset.
  int koff[C::KK];
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk)
    koff[kk] = l32 * (D * 2) + (((2 * kk + g) ^ (l32 & (C::KCH - 1))) * 16);
  // V operand (transposing read): within a 16-lane group G, lane L reads row
  // k0 + L/4 at dv d0 + 4*(L%4), k0 = 16*sg + 8*hh + 4*g, d0 = 32*db + 16*(G&1).
  // The row's swizzle key depends on the row mod 4 = L/4 only, so one base offset
  // per dv block covers every (sg, hh).
  const int G = lane >> 4, L = lane & 15;
  const int vrow = 4 * g + (L >> 2);
  const int vkey = v_swizzle_key(L >> 2) & (C::VCH - 1);
  int voff[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    const int col = 32 * db + 16 * (G & 1) + 4 * (L & 3);
    voff[db] = vrow * (DV * 2) + (((col >> 3) ^ vkey) * 16) + (col & 7) * 2;
  }
  auto vaddr = [&](int sg, int hh, int db) { return (16 * sg + 8 * hh) * (DV * 2) + voff[db]; };
  auto k_operand = [&](const unsigned char* ks, int kk, int kb) {
    return *reinterpret_cast<const e8*>(ks + kb * 32 * (D * 2) + koff[kk]);
  };
  auto v_operand = [&](const unsigned char* vs, int sg, int db) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vs + vaddr(sg, 0, db)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vs + vaddr(sg, 1, db)));
    e8 a;
    a.lo = __builtin_bit_cast(e4, lo);
    a.hi = __builtin_bit_cast(e4, hi);
    return a;
  };

  floatx16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = floatx16{};
  float m_ref = -INFINITY;  // reference (base 2); same in both half-waves
  float l_run = 0.f;        // this half-wave's share of the normaliser

  // S^T(tile) = K Q^T: 2 key blocks x KK dim steps (the two chains alternate).
  auto qk = [&](const unsigned char* ks, floatx16 (&s)[2]) {
    s[0] = floatx16{};
    s[1] = floatx16{};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(k_operand(ks, kk, kb), qreg[kk], s[kb]);
  };
  // O^T += V^T P^T over the tile's 4 groups of 16 keys; dv blocks innermost.
  auto pv = [&](const unsigned char* vs, const e8 (&pk)[4]) {
#pragma unroll
    for (int sg = 0; sg < 4; ++sg)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) oacc[db] = mfma32(v_operand(vs, sg, db), pk[sg], oacc[db]);
  };
  float bcur[BIAS ? 32 : 1];
  auto load_bias = [&](int kv0) {
    if constexpr (BIAS) {
      if (p.bias_vec4 && kv0 + C::BN <= N) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const floatx4 t4 = *reinterpret_cast<const floatx4*>(brow + kv0 + kb * 32 + r4 * 8 + g * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) bcur[kb * 16 + r4 * 4 + e] = t4[e];
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              bcur[kb * 16 + r4 * 4 + e] = brow[min(kv0 + kb * 32 + r4 * 8 + g * 4 + e, N - 1)];
      }
    }
  };
  // Factor from the (biased) score to base-2 logits: without a bias the raw dot
  // product is scaled by log2(e)/sqrt(d); with one, x = s/sqrt(d) + bias is formed
  // first and scaled by log2(e).
  const float cs = BIAS ? kLog2e : p.scale_log2;

  // micro-step k of the softmax of scores s (see SmPlan); writes pk and alpha
  auto sm_step = [&](auto K, SmState& st, floatx16 (&s)[2], e8 (&pk)[4], float& alpha, auto PlanTag,
                     int kv0) {
    using Pl = typename decltype(PlanTag)::type;
    constexpr int k = decltype(K)::value;
    if constexpr (k < Pl::NPRE) {
      s[k / 16][k % 16] = fmaf(s[k / 16][k % 16], p.scale, bcur[k]);
    } else if constexpr (k < Pl::MAX0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key >= N || (p.causal && key > qlim)) s[kb][r] = -INFINITY;
        }
    } else if constexpr (k < Pl::XCH) {
      constexpr int c = (k - Pl::MAX0) & 1, j = (k - Pl::MAX0) >> 1;
      if constexpr (j == 0) st.mx[c] = fmaxf(fmaxf(s[c][0], s[c][1]), s[c][2]);
      else if constexpr (j < 7) st.mx[c] = fmaxf(fmaxf(st.mx[c], s[c][2 * j + 1]), s[c][2 * j + 2]);
      else st.mx[c] = fmaxf(st.mx[c], s[c][15]);
    } else if constexpr (k == Pl::XCH) {
      float bmax = fmaxf(st.mx[0], st.mx[1]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(bmax), __float_as_uint(bmax), false, false);
      bmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * cs;
      // move the reference only when the block max exceeds it by more than kTau
      const bool move = bmax > m_ref + kTau;
      const float new_ref = move ? bmax : m_ref;
      alpha = move ? __builtin_amdgcn_exp2f(m_ref - new_ref) : 1.f;  // exp2(-inf) = 0
      m_ref = new_ref;
      st.nref = (new_ref == -INFINITY) ? 0.f : -new_ref;  // no allowed key yet: add nothing
#pragma unroll
      for (int i = 0; i < 4; ++i) st.ps[i] = 0.f;
    } else if constexpr (k < Pl::UPD) {
      constexpr int e = k - Pl::ELT0;
      if constexpr (e < 32) st.pf[e] = __builtin_amdgcn_exp2f(fmaf(s[e / 16][e % 16], cs, st.nref));
      if constexpr (e >= Pl::LAG) {
        constexpr int f = e - Pl::LAG;
        st.ps[f & 3] += st.pf[f];
        if constexpr (f & 1) {
          constexpr int r = f % 16;
          set_pair(pk[(f / 16) * 2 + r / 8], (r % 8) / 2, cvt_pk<E>(st.pf[f - 1], st.pf[f]));
        }
      }
    } else {
      l_run = alpha * l_run + ((st.ps[0] + st.ps[1]) + (st.ps[2] + st.ps[3]));
    }
  };
  // The general softmax (any tile, with element masks when `edge`): same arithmetic.
  const std::common_type<SmPlan<BIAS>> plain_plan;
  // The general softmax runs its steps back to back, so an exponential's result is
  // used 8 steps later (its latency is not hidden behind matrix instructions here).
  const std::common_type<SmPlan<BIAS, false, 8>> seq_plan;
  auto softmax = [&](floatx16 (&s)[2], e8 (&pk)[4], int kv0, bool edge, float& alpha) {
    using Pl = SmPlan<BIAS, false, 8>;
    SmState st;
    static_for<0, Pl::MAX0>([&](auto K) { sm_step(K, st, s, pk, alpha, seq_plan, kv0); });
    if (edge) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key >= N || (p.causal && key > qlim)) s[kb][r] = -INFINITY;
        }
    }
    static_for<Pl::MAX0, Pl::NOPS>([&](auto K) { sm_step(K, st, s, pk, alpha, seq_plan, kv0); });
  };

  // The steady-state tile body as one fixed sequence of NS slots. The matrix cores
  // first add P(t-1) V(t-1) into o (slots 0 .. NP-1), then form the scores of tile
  // t+1, key block 0 (slots NP .. P2-1) and key block 1 (P2 .. NS-1), into the same
  // registers that hold the scores of tile t; the vector ALUs run the softmax of
  // tile t meanwhile, reading each key block before its registers are overwritten.
  // Slot i issues one matrix instruction, the LDS operand read of the instruction
  // LA slots ahead, and its share of the softmax micro-steps; sched_barrier keeps
  // the compiler from regrouping them.
  auto fused = [&](const unsigned char* ks, const unsigned char* vs, floatx16 (&s)[2], e8 (&pc)[4],
                   const e8 (&pp)[4], float& alpha, int next_kv0) {
    using Pl = SmPlan<BIAS>;
    constexpr int NP = 4 * C::NDB, P2 = NP + C::KK, NS = P2 + C::KK;
    constexpr int LA = 3;  // operand reads run this many slots ahead
    static_assert(Pl::first(NP, NP, P2, NS) >= Pl::ELT0 + 16 && Pl::first(P2, NP, P2, NS) >= Pl::ELT0 + 32,
                  "softmax steps must read each key block before it is overwritten");
    auto operand = [&](auto J) {
      constexpr int j = decltype(J)::value;
      if constexpr (j < NP) return v_operand(vs, j / C::NDB, j % C::NDB);
      else if constexpr (j < P2) return k_operand(ks, j - NP, 0);
      else return k_operand(ks, j - P2, 1);
    };
    e8 ring[LA];
    static_for<0, LA>([&](auto J) { ring[J] = operand(J); });
    SmState st;
    static_for<0, NS>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const e8 a = ring[i % LA];
      if constexpr (i + LA < NS) ring[i % LA] = operand(std::integral_constant<int, i + LA>{});
      // The wave's issue priority is raised for the Q K^T half of the body (the two
      // waves of a SIMD belong to different workgroups and drift in phase; measured
      // 2-6% faster than equal priority, and than raising it for the P V half or around
      // each matrix instruction).
      if constexpr (i == NP) __builtin_amdgcn_s_setprio(1);
      if constexpr (i < NP) {
        oacc[i % C::NDB] = mfma32(a, pp[i / C::NDB], oacc[i % C::NDB]);
      } else {
        constexpr int kb = i < P2 ? 0 : 1, kk = i - (kb ? P2 : NP);
        s[kb] = mfma32(a, qreg[kk], kk == 0 ? floatx16{} : s[kb]);
      }
      static_for<Pl::first(i, NP, P2, NS), Pl::first(i + 1, NP, P2, NS)>(
          [&](auto K) { sm_step(K, st, s, pc, alpha, plain_plan, 0); });
      // the bias of the next tile is loaded as soon as this tile's bias steps are done
      if constexpr (BIAS && Pl::first(i, NP, P2, NS) < Pl::NPRE && Pl::first(i + 1, NP, P2, NS) >= Pl::NPRE)
        load_bias(next_kv0);
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_setprio(0);
  };

  // A wave's last tile (no next scores to form; the causal diagonal tile, or the
  // last tile of its key range): P(t-1) V(t-1) on the matrix cores while the vector
  // ALUs run the softmax of tile t, element masks included when EDGE.
  auto fused_last = [&](const unsigned char* vs, floatx16 (&s)[2], e8 (&pc)[4], const e8 (&pp)[4],
                        float& alpha, int kv0, auto EDGEc) {
    constexpr bool EDGE = decltype(EDGEc)::value;
    using Pl = SmPlan<BIAS, EDGE>;
    const std::common_type<Pl> plan;
    constexpr int NP = 4 * C::NDB;
    constexpr int LA = 3;
    auto operand = [&](auto J) {
      constexpr int j = decltype(J)::value;
      return v_operand(vs, j / C::NDB, j % C::NDB);
    };
    e8 ring[LA];
    static_for<0, LA>([&](auto J) { ring[J] = operand(J); });
    SmState st;
    static_for<0, NP>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const e8 a = ring[i % LA];
      if constexpr (i + LA < NP) ring[i % LA] = operand(std::integral_constant<int, i + LA>{});
      oacc[i % C::NDB] = mfma32(a, pp[i / C::NDB], oacc[i % C::NDB]);
      static_for<Pl::first(i, NP, NP, NP), Pl::first(i + 1, NP, NP, NP)>(
          [&](auto K) { sm_step(K, st, s, pc, alpha, plan, kv0); });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  TileCopy<D, C::KLD, false> kcp;
  TileCopy<DV, C::VLD, true> vcp;
  kcp.init(p.k_sn, wave, lane);
  vcp.init(p.v_sn, wave, lane);
  auto copy_k = [&](unsigned char* st, int t) { kcp.copy(st, tile_rsrc(kp, p.k_sn, t * C::BN, N), wave); };
  auto copy_v = [&](unsigned char* st, int t) { vcp.copy(st, tile_rsrc(vp, p.v_sn, t * C::BN, N), wave); };

  // ---- prologue: K(t_begin), K(t_begin+1) into LDS; scores of t_begin ----
  // Vector-memory loads complete in issue order, so waiting until only the last KLD
  // loads (K(t_begin+1)) are outstanding means Q and K(t_begin) have landed; K(t_begin+1)
  // keeps arriving while the first scores are formed (the first loop step waits for it).
  copy_k(k_lds0, t_begin);
  if (t_begin + 1 < t_end) {
    copy_k(k_lds1, t_begin + 1);
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(C::KLD));
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();

  // Iteration t (stage parity PAR = (t - t_begin) mod 2): the matrix cores add
  // P(t-1) V(t-1) into o and compute the scores of tile t+1 while the vector ALUs run
  // the softmax of tile t; the copies of K(t+2) and V(t) are in flight meanwhile. K(t)
  // and V(t) live in stage PAR. `s` holds the scores of tile t on entry and of tile
  // t+1 on exit; `pc`/`pp` hold the bf16 probabilities of tiles t and t-1, and the
  // caller swaps their roles every iteration, so no register copies are needed. o is
  // rescaled by alpha(t-1) before P(t-1) V(t-1) is added.
  float alpha_prev = 1.f;
  auto step = [&](auto PARc, int t, floatx16 (&s)[2], e8 (&pc)[4], const e8 (&pp)[4]) {
    constexpr int PAR = decltype(PARc)::value;
    unsigned char* k_same = PAR ? k_lds1 : k_lds0;   // K(t), refilled with K(t+2)
    unsigned char* k_next = PAR ? k_lds0 : k_lds1;   // K(t+1)
    unsigned char* v_same = PAR ? v_lds1 : v_lds0;   // filled with V(t)
    unsigned char* v_prev = PAR ? v_lds0 : v_lds1;   // V(t-1)
    // K(t+1) and V(t-1) have landed for every wave, and no wave still reads the stages
    // refilled below (K(t) was read for the scores of tile t, V(t-2) by P V of t-2)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < t_end) copy_k(k_same, t + 2);
    if (t < t_end) copy_v(v_same, t);
    const int kv0 = t * C::BN;
    const bool do_qk = t + 1 < tw_end;
    const bool do_sm = t < tw_end;
    const bool do_pv = t > t_begin && t - 1 < tw_end;
    const bool edge = (kv0 + C::BN > N) || (p.causal && kv0 + C::BN - 1 > wq0 + p.coff);
    if (do_pv && __builtin_amdgcn_ballot_w64(alpha_prev != 1.f)) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) oacc[db] *= alpha_prev;
    }
    float alpha = 1.f;
    if (do_qk && do_sm && do_pv && !edge) {
      fused(k_next, v_prev, s, pc, pp, alpha, kv0 + C::BN);
    } else if (!do_qk && do_sm && do_pv) {
      if (edge) fused_last(v_prev, s, pc, pp, alpha, kv0, std::true_type{});
      else fused_last(v_prev, s, pc, pp, alpha, kv0, std::false_type{});
    } else {
      if (do_sm) softmax(s, pc, kv0, edge, alpha);
      if constexpr (BIAS) {
        if (t + 1 < tw_end) load_bias(kv0 + C::BN);  // the bias of tile t+1, one tile ahead
      }
      if (do_qk) qk(k_next, s);
      if (do_pv) pv(v_prev, pp);
    }
    alpha_prev = alpha;
  };
  floatx16 s[2];
  e8 pA[4], pB[4];
  if (t_begin < tw_end) qk(k_lds0, s);
  if constexpr (BIAS) {
    if (t_begin < tw_end) load_bias(t_begin * C::BN);
  }
  for (int t = t_begin; t <= t_end; t += 2) {
    step(std::integral_constant<int, 0>{}, t, s, pA, pB);
    if (t + 1 <= t_end) step(std::integral_constant<int, 1>{}, t + 1, s, pB, pA);
  }

  // ---- epilogue ----
  // register r of dv block db holds dv = db*32 + (r/4)*8 + g*4 + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int row = wave * 32 + l32;  // row within the query tile

  if (!U.partial) {
    if (!qvalid) return;
    E* op = static_cast<E*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)qi * p.o_sn;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        e4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (E)(oacc[db][r4 * 4 + e] * inv);
        *reinterpret_cast<e4*>(op + db * 32 + r4 * 8 + g * 4) = o4;
      }
    if (p.lse && g == 0)
      p.lse[b * p.l_sb + h * p.l_sh + qi] = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    return;
  }

  // ---- split: this range's partial state: its own normalised output o / l in bf16
  // (a convex combination of V rows, so the rounding costs at most 2^-9 max|v|, that of
  // the bf16 output itself, and equal V rows come back exactly), layout per slot
  // [BM/32][dv/4][32][4]: one wave's 32 rows of 4 dv values are 256 consecutive bytes;
  // m and l stay fp32. ----
  const __amdgpu_buffer_rsrc_t po = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<E*>(p.part_o) + (int64_t)U.slot * (C::BM * DV), 0, C::BM * DV * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t pml = __builtin_amdgcn_make_buffer_rsrc(
      p.part_ml + (int64_t)U.slot * (2 * C::BM), 0, 2 * C::BM * 4, kBufferWord3);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // a wave whose rows all lie past the last query row stores nothing (no merge reads it)
  if (wq0 < p.Nq) {
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c4 = db * 8 + r4 * 2 + g;
      e4 h4;
#pragma unroll
      for (int e = 0; e < 4; ++e) h4[e] = (E)(oacc[db][r4 * 4 + e] * inv);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h4), po,
                                            ((wave * (DV / 4) + c4) * 32 + l32) * 8, 0, kStoreWriteThrough);
    }
  if (g == 0) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_ref), pml, row * 4, 0, kStoreWriteThrough);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_tot), pml, (C::BM + row) * 4, 0, kStoreWriteThrough);
  }
  }
  if (p.part_flag) {  // merged by merge blocks of this kernel: publish the state
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores are complete (written through)
    __syncthreads();
    if (tid == 0) __hip_atomic_store(p.part_flag + U.slot, p.seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Every variant is instantiated explicitly: the host pass then emits a launch stub
// for each of them (implicit instantiation through the launch macro alone left all
// but one of them undefined with this compiler).
#define FA_FWD_VARIANTS(E)                                   \
  template __global__ void fwd_mfma<E, 64, 64, false>(Params);  \
  template __global__ void fwd_mfma<E, 64, 64, true>(Params);   \
  template __global__ void fwd_mfma<E, 64, 128, false>(Params); \
  template __global__ void fwd_mfma<E, 64, 128, true>(Params);  \
  template __global__ void fwd_mfma<E, 128, 64, false>(Params); \
  template __global__ void fwd_mfma<E, 128, 64, true>(Params);  \
  template __global__ void fwd_mfma<E, 128, 128, false>(Params);\
  template __global__ void fwd_mfma<E, 128, 128, true>(Params); \
  template __global__ void merge_split<E, 64>(Params);          \
  template __global__ void merge_split<E, 128>(Params);
FA_FWD_VARIANTS(__bf16)
FA_FWD_VARIANTS(_Float16)
#undef FA_FWD_VARIANTS

template <typename E, int D, int DV>
hipError_t launch_dd(const Params& p, int grid, bool merge, hipStream_t stream) {
  if (p.bias)
    FA_LAUNCH_MAIN((fwd_mfma<E, D, DV, true>), dim3(grid), dim3(256), stream, p);
  else
    FA_LAUNCH_MAIN((fwd_mfma<E, D, DV, false>), dim3(grid), dim3(256), stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !merge) return e;
  hipLaunchKernelGGL((merge_split<E, DV>), dim3(merge_groups(DV, 1), p.B * p.H, p.n_split), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const Params& p, int grid, bool merge, hipStream_t stream) {
  if (p.d == 128 && p.dv == 128) return launch_dd<E, 128, 128>(p, grid, merge, stream);
  if (p.d == 64 && p.dv == 128) return launch_dd<E, 64, 128>(p, grid, merge, stream);
  if (p.d == 128 && p.dv == 64) return launch_dd<E, 128, 64>(p, grid, merge, stream);
  if (p.d == 64 && p.dv == 64) return launch_dd<E, 64, 64>(p, grid, merge, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_mfma(const Params& p, int grid, bool merge, bool fp16, hipStream_t stream) {
  return fp16 ? launch_e<_Float16>(p, grid, merge, stream) : launch_e<__bf16>(p, grid, merge, stream);
}

}  // namespace fa

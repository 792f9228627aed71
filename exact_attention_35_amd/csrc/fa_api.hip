// Host side of the C ABI declared in include/fa.h, include/fa_bwd.h and
// include/fa_plan.h: argument validation, the work plan (query tiles and key splits),
// scratch workspaces, and kernel dispatch.
//
// The contract follows the page "编译器与内核" (Compilers and kernels): a kernel
// implements a bounded contract over shapes, strides, dtype, layout, aliasing,
// mutation, numerics and target (section "内核实现一份有边界的契约"), so every fact the
// kernels rely on is checked here before anything is enqueued; and a library's
// contract covers dtype, layout, workspace, determinism and stream semantics
// (section "生态系统也是目标的一部分").
//
// Validation is plain host arithmetic and makes no HIP call, so an invalid call
// returns its status without touching the device.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <random>
#include <utility>
#include <vector>

#include "fa.h"
#include "fa_bwd.h"
#include "fa_plan.h"
#include "fa_internal.h"

namespace {

using fa::Params;

constexpr int kMaxSplitBH = 64;  // split plans: b*h fits the unit table's 6-bit field
constexpr int kMaxSplitBH1 = 1 << 14;  // ... and its 14 bits when there is one query tile
constexpr int64_t kMaxRowStride = 1 << 24;     // bf16 k/v row stride limit (elements)

struct Range {
  uintptr_t lo, hi;  // [lo, hi) in bytes
};

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// Byte range touched by a tensor with sizes n[0..nd) and strides s[0..nd) (elements)
// plus a contiguous innermost axis of `inner` elements.
Range extent(const void* base, const int64_t* n, const int64_t* s, int nd, int64_t inner, int elem) {
  int64_t last = inner - 1;
  for (int i = 0; i < nd; ++i) last += (n[i] - 1) * s[i];
  const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
  return Range{lo, lo + (uintptr_t)((last + 1) * elem)};
}

// True when distinct (index tuple, inner offset) pairs map to distinct addresses.
bool non_overlapping(const int64_t* n, const int64_t* s, int nd, int64_t inner) {
  std::pair<int64_t, int64_t> dims[4];
  int k = 0;
  for (int i = 0; i < nd; ++i)
    if (n[i] > 1) dims[k++] = {s[i], n[i]};
  std::sort(dims, dims + k);
  int64_t span = inner;  // elements spanned so far
  for (int i = 0; i < k; ++i) {
    if (dims[i].first < span) return false;
    span = dims[i].first * (dims[i].second - 1) + span;
  }
  return true;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Problem {
  const void *q, *k, *v;
  const float* bias;
  void* out;
  float* lse;
  int64_t B, H, N, d, dv;  // N: keys (rows of K, V)
  int64_t Nq;              // query rows (rows of Q, O, lse)
  int mask, dtype;
  fa_strides st;
};

fa_strides contiguous_strides(int64_t H, int64_t Nq, int64_t N, int64_t d, int64_t dv) {
  fa_strides s;
  s.q[0] = H * Nq * d; s.q[1] = Nq * d; s.q[2] = d;
  s.k[0] = H * N * d; s.k[1] = N * d; s.k[2] = d;
  s.v[0] = H * N * dv; s.v[1] = N * dv; s.v[2] = dv;
  s.out[0] = H * Nq * dv; s.out[1] = Nq * dv; s.out[2] = dv;
  s.bias[0] = H * Nq * N; s.bias[1] = Nq * N; s.bias[2] = N;
  s.lse[0] = H * Nq; s.lse[1] = Nq;
  return s;
}

bool supported_width(int64_t x) { return x >= 1 && x <= 256; }
bool mfma_width(int64_t x) { return x == 64 || x == 128; }
int elem_size(int dtype) { return dtype == FA_F32 ? 4 : 2; }

// Size/shape/dtype/mask checks shared by the size queries and the forward calls
// (Nq query rows against N keys).
int check_shape_qk(int64_t B, int64_t H, int64_t Nq, int64_t N, int64_t d, int64_t dv, int dtype, int mask) {
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (B < 0 || H < 0 || N < 0 || Nq < 0) return FA_ERR_SHAPE;
  if (!supported_width(d) || !supported_width(dv)) return FA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 30;
  if (B > lim || H > lim || N > lim || Nq > lim) return FA_ERR_SHAPE;
  if (B * H > lim || (B * H) * ((std::max(N, Nq) + 63) / 64) > lim) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype, int mask) {
  return check_shape_qk(B, H, N, N, d, dv, dtype, mask);
}

int validate(const Problem& P) {
  int st = check_shape_qk(P.B, P.H, P.Nq, P.N, P.d, P.dv, P.dtype, P.mask);
  if (st != FA_OK) return st;
  if (P.B * P.H * P.Nq == 0) return FA_OK;  // no output rows: nothing to do
  if (!P.q || !P.out || (P.N > 0 && (!P.k || !P.v))) return FA_ERR_NULL;
  const fa_strides& s = P.st;
  const int64_t* all[] = {s.q, s.k, s.v, s.out, s.bias};
  for (int t = 0; t < 5; ++t)
    for (int i = 0; i < 3; ++i)
      if (all[t][i] < 0) return FA_ERR_STRIDE;
  if (s.lse[0] < 0 || s.lse[1] < 0) return FA_ERR_STRIDE;
  const int64_t sz[3] = {P.B, P.H, P.Nq};   // q, out, lse, bias rows
  const int64_t szk[3] = {P.B, P.H, P.N};   // k, v
  if (!non_overlapping(sz, s.out, 3, P.dv)) return FA_ERR_STRIDE;
  if (P.lse && !non_overlapping(sz, s.lse, 2, P.Nq)) return FA_ERR_STRIDE;

  const int es = elem_size(P.dtype);
  const void* ptrs[4] = {P.q, P.k, P.v, P.out};
  for (int t = 0; t < 4; ++t)
    if (!aligned(ptrs[t], es)) return FA_ERR_ALIGN;
  if (P.bias && !aligned(P.bias, 4)) return FA_ERR_ALIGN;
  if (P.lse && !aligned(P.lse, 4)) return FA_ERR_ALIGN;

  // aliasing: outputs must not overlap inputs or each other
  const Range rq = extent(P.q, sz, s.q, 3, P.d, es);
  const Range rk = P.N ? extent(P.k, szk, s.k, 3, P.d, es) : Range{0, 0};
  const Range rv = P.N ? extent(P.v, szk, s.v, 3, P.dv, es) : Range{0, 0};
  const Range ro = extent(P.out, sz, s.out, 3, P.dv, es);
  if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv)) return FA_ERR_ALIAS;
  Range rb{0, 0};
  if (P.bias && P.N) {
    rb = extent(P.bias, sz, s.bias, 3, P.N, 4);
    if (overlaps(ro, rb)) return FA_ERR_ALIAS;
  }
  if (P.lse) {
    const Range rl = extent(P.lse, sz, s.lse, 2, P.Nq, 4);
    if (overlaps(rl, rq) || overlaps(rl, rk) || overlaps(rl, rv) || overlaps(rl, ro)) return FA_ERR_ALIAS;
    if (P.bias && overlaps(rl, rb)) return FA_ERR_ALIAS;
  }
  return FA_OK;
}

// ---------------------------------------------------------------- device facts
struct DevInfo {
  bool probed = false;
  bool gfx950 = false;
  int cus = 0;
};
std::mutex g_dev_mu;
DevInfo g_dev[64];

int device_info(int* dev_out, DevInfo* info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return FA_ERR_DEVICE;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo& di = g_dev[dev];
  if (!di.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
    di.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    di.cus = prop.multiProcessorCount;
    di.probed = true;
  }
  *dev_out = dev;
  *info = di;
  return di.gfx950 ? FA_OK : FA_ERR_DEVICE;
}

// ---------------------------------------------------------------- work plan
struct Plan {
  bool mfma = false;
  int n_qt = 0;
  bool split = false;   // query tiles cut into key ranges (units) merged afterwards
  int shift = 0;        // range boundaries in granules of 2^shift key tiles
  struct Ranges {       // the key ranges of one query tile
    int nch;
    int begin[fa::kMaxRanges], len[fa::kMaxRanges];
  };
  Ranges ranges[fa::kMaxSplitQTiles];
  int grid = 0;         // forward workgroups (units)
  int merge_grid = 0;   // blocks of a separate merge kernel (0: no split query tile)
  int merge_blocks = 0; // merge blocks appended to the forward grid instead
  size_t ws_bytes = 0;
  size_t off_flag = 0, off_ml = 0, off_o = 0;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int env_int(const char* name) {
  const char* e = std::getenv(name);
  return e ? std::atoi(e) : 0;
}

// Key tiles of query tile qt (causal tiles stop at the last key the tile's last row may
// see, qt*BM + BM - 1 + coff; coff = N - Nq).
int64_t qtile_ntiles(int64_t N, int64_t coff, int qt, bool causal) {
  const int64_t bm = fa::kMfmaBM, bn = fa::kMfmaBN;
  const int64_t kv = causal ? std::min(N, (qt + 1) * bm + coff) : N;
  return (std::max<int64_t>(kv, 0) + bn - 1) / bn;
}

// Cost model of the split plans, in key tiles: the second workgroup on a CU runs its
// tiles about 1.3x slower than the first while both run (the older waves issue first),
// and the range holding a causal query tile's diagonal costs about 1.5 tiles more
// (masked tiles; half the waves stop one tile earlier). Units 0 .. cus-1 are the first
// workgroups of their CUs.
constexpr double kSecondSlotCost = 1.3;
constexpr double kDiagonalCost = 1.5;

// Cuts nt key tiles into nch consecutive ranges of about equal cost for units u0 ..
// u0+nch-1 (range k costs len_k * c_k, plus the diagonal cost for the last range);
// returns the largest range cost. Range boundaries fall on multiples of G key tiles (the
// granule of the unit table's fields); nch is at most ceil(nt / G).
double cut_even(int nt, int nch, int64_t u0, int cus, double diag, int G, Plan::Ranges* r) {
  double c[fa::kMaxRanges], inv_sum = 0.0, extra = 0.0;
  for (int k = 0; k < nch; ++k) {
    c[k] = u0 + k < cus ? 1.0 : kSecondSlotCost;
    inv_sum += 1.0 / c[k];
  }
  extra = diag / c[nch - 1];
  const double T = (nt + extra) / inv_sum;  // the common cost if tiles were divisible
  const int ng = (nt + G - 1) / G;          // granules
  int tg = 0;
  double acc = 0.0, worst = 0.0;
  for (int k = 0; k < nch; ++k) {
    acc += T / c[k] - (k == nch - 1 ? extra : 0.0);
    int endg = k == nch - 1 ? ng : (int)std::lround(acc / G);
    endg = std::min(std::max(endg, tg + 1), ng - (nch - 1 - k));  // every range keeps >= 1 granule
    r->begin[k] = tg * G;
    r->len[k] = std::min(endg * G, nt) - tg * G;
    worst = std::max(worst, r->len[k] * c[k] + (k == nch - 1 ? diag : 0.0));
    tg = endg;
  }
  r->nch = nch;
  return worst;
}

// Cuts every query tile, from the last one, into the fewest equal-cost ranges whose
// cost is at most `cap`. Returns the number of units, or -1 when a tile would need more
// than kMaxRanges ranges.
int64_t cut_ranges(const Plan& pl, int64_t N, int64_t coff, int64_t BH, bool causal, int cus, double cap,
                   Plan::Ranges* out) {
  const int G = 1 << pl.shift;
  int64_t u = 0;
  for (int qt = pl.n_qt - 1; qt >= 0; --qt) {
    const int nt = (int)qtile_ntiles(N, coff, qt, causal);
    if (nt == 0) {  // rows that see no key: one unit writes O = 0 and lse = -inf
      out[qt].nch = 1;
      out[qt].begin[0] = 0;
      out[qt].len[0] = 0;
      u += BH;
      continue;
    }
    const int ng = (nt + G - 1) / G;
    const double diag = causal ? kDiagonalCost : 0.0;
    int nch = 1;
    while (cut_even(nt, nch, u, cus, diag, G, &out[qt]) > cap && nch < std::min(ng, fa::kMaxRanges)) ++nch;
    if (cut_even(nt, nch, u, cus, diag, G, &out[qt]) > cap && nch < ng) return -1;
    u += BH * nch;
  }
  return u;
}

// Widest field of the unit table: first key tile and key-tile count are 9 bits each.
constexpr int kUnitFieldMax = 511;

// One unit table entry: query tile (bits 0-7), first key tile (8-16) and key-tile count
// (17-25), both in granules of 2^shift tiles (the count rounded up: the kernel clips the
// last range of a tile to the tile's key tiles), b*h (26-31). Plans with a single query
// tile put b*h's low 8 bits in bits 0-7.
uint32_t pack_unit(int qt, int begin, int len, int64_t bh, bool one_qtile, int shift) {
  const uint32_t lo = one_qtile ? (uint32_t)(bh & 0xff) : (uint32_t)qt;
  const uint32_t hi = one_qtile ? (uint32_t)(bh >> 8) : (uint32_t)bh;
  const uint32_t b = (uint32_t)(begin >> shift), n = (uint32_t)((len + (1 << shift) - 1) >> shift);
  return lo | b << 8 | n << 17 | hi << 26;
}

// Merge blocks per split tile and b*h: the row groups of a query tile that hold query
// rows (all of them unless the only tile is short, as in decoding).
int merge_groups_used(int64_t Nq, int n_qt, int64_t dv) {
  const int groups = fa::merge_groups((int)dv, fa::kFusedMergeItems);
  const int rows = fa::kMfmaBM / groups;
  return n_qt == 1 ? (int)std::min<int64_t>(groups, (Nq + rows - 1) / rows) : groups;
}

Plan make_plan(int64_t B, int64_t H, int64_t Nq, int64_t N, int64_t d, int64_t dv, int dtype, int mask, int cus) {
  Plan pl;
  pl.mfma = (dtype == FA_BF16 || dtype == FA_F16) && mfma_width(d) && mfma_width(dv);
  if (!pl.mfma) return pl;
  const bool causal = mask == FA_MASK_CAUSAL;
  const int64_t coff = N - Nq;
  const int bm = fa::kMfmaBM;
  pl.n_qt = (int)((Nq + bm - 1) / bm);
  const int64_t BH = B * H;
  const int64_t tiles = BH * pl.n_qt;
  pl.grid = (int)tiles;
  // Split where the query tiles do not give every CU two workgroups (below one per CU
  // CUs idle; below two, a causal problem's longest tiles set the time: measured
  // 147 -> 84 us for four causal heads of 8192) and the unit table's fields fit
  // (b*h < 64, or < 2^14 with one query tile; query tile < 256).
  if (tiles <= 0 || tiles >= 2 * (int64_t)cus || BH > (pl.n_qt == 1 ? kMaxSplitBH1 : kMaxSplitBH) ||
      pl.n_qt > fa::kMaxSplitQTiles)
    return pl;
  // The first key tile and the tile count of a unit are stored in granules of 2^shift
  // key tiles, the smallest granule for which the longest query tile's key tiles fit the
  // 9-bit fields (shift 0 up to 32704 keys per query tile).
  int64_t nt_max = 0;
  for (int qt = 0; qt < pl.n_qt; ++qt) nt_max = std::max(nt_max, qtile_ntiles(N, coff, qt, causal));
  while (((nt_max + (1 << pl.shift) - 1) >> pl.shift) > kUnitFieldMax) ++pl.shift;
  if (pl.shift > 15) {
    pl.shift = 0;
    return pl;
  }
  // Cut the query tiles' key ranges into units of about equal cost, as many as the CUs
  // hold at once (two workgroups per CU): the smallest cost cap whose cut fits.
  const int64_t target = std::min<int64_t>(fa::kMaxSplitUnits,
                                           env_int("FA_SPLIT_UNITS") > 0 ? env_int("FA_SPLIT_UNITS") : 2 * (int64_t)cus);
  double lo = 0.5, hi = (double)nt_max * kSecondSlotCost + kDiagonalCost + 1.0;
  if (cut_ranges(pl, N, coff, BH, causal, cus, hi, pl.ranges) < 0) return pl;
  for (int it = 0; it < 24; ++it) {
    const double mid = 0.5 * (lo + hi);
    const int64_t u = cut_ranges(pl, N, coff, BH, causal, cus, mid, pl.ranges);
    if (u >= 0 && u <= target) hi = mid;
    else lo = mid;
  }
  const int64_t units = cut_ranges(pl, N, coff, BH, causal, cus, hi, pl.ranges);
  int64_t n_split = 0;
  for (int qt = 0; qt < pl.n_qt; ++qt) n_split += pl.ranges[qt].nch > 1;
  if (n_split == 0) return pl;
  pl.split = true;
  pl.grid = (int)units;
  pl.merge_grid = (int)(n_split * BH * fa::merge_groups((int)dv, 1));
  pl.merge_blocks = (int)(n_split * BH * merge_groups_used(Nq, pl.n_qt, dv));
  pl.off_flag = 0;
  pl.off_ml = round_up(units * sizeof(uint64_t), 256);
  pl.off_o = round_up(pl.off_ml + units * 2 * bm * sizeof(float), 256);
  pl.ws_bytes = round_up(pl.off_o + (size_t)units * bm * dv * 2, 256);  // bf16 numerators
  return pl;
}

// The plan of a problem depends only on its shape and the CU count; cutting the ranges
// of a split plan takes a while on the host, so plans are kept (a bounded map; a
// caller holds its plan by shared pointer, so clearing the map never frees one in use).
std::shared_ptr<const Plan> cached_plan(int64_t B, int64_t H, int64_t Nq, int64_t N, int64_t d, int64_t dv,
                                        int dtype, int mask, int cus) {
  using Key = std::array<int64_t, 9>;
  static std::mutex mu;
  static std::map<Key, std::shared_ptr<const Plan>> cache;
  const Key key{B, H, Nq, N, d, dv, dtype, mask, cus};
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  auto pl = std::make_shared<const Plan>(make_plan(B, H, Nq, N, d, dv, dtype, mask, cus));
  std::lock_guard<std::mutex> lk(mu);
  if (cache.size() >= 256) cache.clear();
  cache.emplace(key, pl);
  return pl;
}

// ---------------------------------------------------------------- launch
bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();  // not ours to report; take the path that is safe under capture
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

// A number unique to each call (odd, so never the zero of fresh memory), published by
// the units of an in-kernel merge. It starts at a random value, so flags left in a
// workspace by other calls or processes do not match it.
uint64_t next_call_number() {
  static std::atomic<uint64_t> next{[] {
    std::random_device rd;
    const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    return ((((uint64_t)rd() << 32) ^ rd()) ^ (t * 0x9E3779B97F4A7C15ull)) | 1ull;
  }()};
  return next.fetch_add(2, std::memory_order_relaxed);
}

// The matrix-core kernel's layout conditions (checked per call; the plan depends on the
// shape only): 16-byte aligned bases and row strides of q, k, v and out (128-bit loads
// and stores), and k/v row strides below 2^24 elements (a 64-row tile is addressed
// with 32-bit byte offsets). Other layouts take the general kernel.
bool mfma_layout_ok(const Problem& P) {
  const fa_strides& s = P.st;
  const void* ptrs[4] = {P.q, P.k, P.v, P.out};
  const int64_t* strd[4] = {s.q, s.k, s.v, s.out};
  for (int t = 0; t < 4; ++t) {
    if (!aligned(ptrs[t], 16)) return false;
    for (int i = 0; i < 3; ++i)
      if ((strd[t][i] * 2) % 16 != 0) return false;
  }
  return s.k[2] < kMaxRowStride && s.v[2] < kMaxRowStride;
}

int run(const Problem& P, const Plan& pl_in, void* ws, hipStream_t stream) {
  // a shape planned for the matrix cores whose layout is not theirs runs on the
  // general kernel (no split; the workspace is then unused)
  static const Plan kGenericPlan{};
  const Plan& pl = pl_in.mfma && !mfma_layout_ok(P) ? kGenericPlan : pl_in;
  Params p{};
  p.q = P.q; p.k = P.k; p.v = P.v; p.bias = P.bias; p.out = P.out; p.lse = P.lse;
  const fa_strides& s = P.st;
  p.q_sb = s.q[0]; p.q_sh = s.q[1]; p.q_sn = s.q[2];
  p.k_sb = s.k[0]; p.k_sh = s.k[1]; p.k_sn = s.k[2];
  p.v_sb = s.v[0]; p.v_sh = s.v[1]; p.v_sn = s.v[2];
  p.o_sb = s.out[0]; p.o_sh = s.out[1]; p.o_sn = s.out[2];
  p.b_sb = s.bias[0]; p.b_sh = s.bias[1]; p.b_si = s.bias[2];
  p.l_sb = s.lse[0]; p.l_sh = s.lse[1];
  p.B = (int)P.B; p.H = (int)P.H; p.N = (int)P.N; p.d = (int)P.d; p.dv = (int)P.dv;
  p.Nq = (int)P.Nq;
  p.coff = (int)(P.N - P.Nq);
  p.causal = P.mask == FA_MASK_CAUSAL;
  p.bias_vec4 = P.bias && aligned(P.bias, 16) && s.bias[0] % 4 == 0 && s.bias[1] % 4 == 0 && s.bias[2] % 4 == 0;
  // tile shape of the general fp32 kernel for the tile-shape experiment (FA_GENERIC_TILE
  // 1..4; 0, the default, is 64 rows x 32 keys)
  p.gtile = env_int("FA_GENERIC_TILE");
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.d));
  p.scale = (float)(1.0 / std::sqrt((double)P.d));
  p.n_qt = pl.n_qt;
  p.split = pl.split;
  if (pl.split) {  // unit table of the split plan (query tiles from the last)
    int32_t acc = 0;
    int n_split = 0;
    for (int qt = pl.n_qt - 1; qt >= 0; --qt) {
      const Plan::Ranges& r = pl.ranges[qt];
      if (r.nch > 1) p.split_info[n_split++] = fa::split_word(acc, r.nch, qt);
      for (int64_t bh = 0; bh < P.B * P.H; ++bh)
        for (int c = 0; c < r.nch; ++c)
          p.unit_info[acc + bh * r.nch + c] = pack_unit(qt, r.begin[c], r.len[c], bh, pl.n_qt == 1, pl.shift);
      acc += (int32_t)(P.B * P.H * r.nch);
    }
    p.n_split = n_split;
  }
  // Split query tiles are merged by blocks appended to the forward grid, except under
  // graph capture (a replay would reuse this call's number, so the flags of the previous
  // replay would already match): there a separate merge kernel follows.
  const bool split = pl.split;
  const bool in_kernel_merge = split && !stream_capturing(stream) && env_int("FA_MERGE_KERNEL") == 0;
  p.n_units = pl.grid;
  p.unit_shift = pl.shift;
  p.merge_groups = merge_groups_used(P.Nq, pl.n_qt, P.dv);
  p.seq = next_call_number();
  if (pl.ws_bytes > 0) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    p.part_flag = in_kernel_merge ? reinterpret_cast<uint64_t*>(w + pl.off_flag) : nullptr;
    p.part_ml = reinterpret_cast<float*>(w + pl.off_ml);
    p.part_o = w + pl.off_o;
  }
  const int grid = pl.grid + (in_kernel_merge ? pl.merge_blocks : 0);
  hipError_t e = pl.mfma ? fa::launch_mfma(p, grid, split && !in_kernel_merge, P.dtype == FA_F16, stream)
                         : fa::launch_generic(p, P.dtype, stream);
  if (std::getenv("FA_LOG"))
    std::fprintf(stderr, "[fa] %s B=%lld H=%lld Nq=%lld N=%lld d=%lld dv=%lld causal=%d bias=%d n_qt=%d split=%d grid=%d merge=%d ws=%zu\n",
                 pl.mfma ? (P.dtype == FA_F16 ? "mfma_f16" : "mfma_bf16")
                         : (P.dtype == FA_BF16 ? "generic_bf16" : P.dtype == FA_F16 ? "generic_f16" : "generic_f32"),
                 (long long)P.B, (long long)P.H, (long long)P.Nq, (long long)P.N, (long long)P.d, (long long)P.dv,
                 p.causal, P.bias != nullptr, pl.n_qt, (int)pl.split, grid, pl.merge_grid, pl.ws_bytes);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

Problem make_problem(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
                     void* out, float* lse, int64_t B, int64_t H, int64_t Nq, int64_t N, int64_t d, int64_t dv,
                     const fa_strides* strides, int dtype) {
  Problem P;
  P.q = q; P.k = k; P.v = v; P.bias = bias; P.out = out; P.lse = lse;
  P.B = B; P.H = H; P.N = N; P.Nq = Nq; P.d = d; P.dv = dv; P.mask = mask_mode; P.dtype = dtype;
  P.st = strides ? *strides : contiguous_strides(H, Nq, N, d, dv);
  return P;
}

// ---------------------------------------------------------------- owned workspaces
// One library-owned scratch buffer per (device, stream), shared by fa_fwd and fa_bwd
// (calls on one stream run in order, so they never use it at the same time). It only
// grows: a larger need allocates a new buffer and retires the old one, which stays
// allocated until fa_shutdown(), so a pointer handed to a call (maybe on another host
// thread, not yet enqueued) is never freed under it. While the stream captures a graph
// nothing is allocated: a call that would need to allocate returns FA_ERR_WORKSPACE,
// and so does any call that needs scratch memory at all (a graph would keep using the
// shared buffer on every replay); captured work takes the _ex entry points.
struct OwnedWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, OwnedWs> g_ws;
std::vector<std::pair<int, void*>> g_ws_retired;  // (device, buffer), freed by fa_shutdown

int owned_workspace(int dev, hipStream_t stream, size_t need, void** out) {
  if (stream_capturing(stream)) return FA_ERR_WORKSPACE;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  OwnedWs& w = g_ws[{dev, stream}];
  if (w.bytes < need) {
    const size_t grow = std::max(need, w.bytes + w.bytes / 2);
    void* p = nullptr;
    if (hipMalloc(&p, grow) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_ALLOC;
    }
    if (w.ptr) g_ws_retired.emplace_back(dev, w.ptr);
    w.ptr = p;
    w.bytes = grow;
  }
  *out = w.ptr;
  return FA_OK;
}

// ---------------------------------------------------------------- static scratch
// Scratch memory of fa_fwd_qk_noalloc: a fixed device array per GPU (each device that
// loads this library holds its own copy until the process ends). The largest forward
// plan needs kMaxSplitUnits units of dv = 128: 8-byte flags, 2 * 128 fp32 row
// statistics and 128 * 128 16-bit partial outputs per unit, each part 256-byte aligned.
constexpr size_t kStaticScratchBytes =
    ((size_t)fa::kMaxSplitUnits * 8 + 255) / 256 * 256 + (size_t)fa::kMaxSplitUnits * 2 * fa::kMfmaBM * 4 +
    (size_t)fa::kMaxSplitUnits * fa::kMfmaBM * 128 * 2;
static_assert(kStaticScratchBytes % 256 == 0, "scratch parts are 256-byte aligned");
static_assert(kStaticScratchBytes == FA_NOALLOC_SCRATCH_BYTES, "fa.h states the scratch size");

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};  // device address of `scratch` per device (host-side name is not it)

// The device address of this device's `scratch`, looked up once per device with the
// device current (the caller's current device is the one fa_fwd_qk_noalloc runs on).
int static_scratch(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return FA_ERR_DEVICE;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

// ---------------------------------------------------------------- gradients
struct BwdProblem {
  const void *q, *k, *v, *out, *dout;
  const float* lse;
  const float* bias;
  void *dq, *dk, *dv;
  int64_t B, H, N, d, dvw;
  int mask, dtype;
  fa_bwd_strides st;
};

fa_bwd_strides contiguous_bwd_strides(int64_t H, int64_t N, int64_t d, int64_t dv) {
  fa_bwd_strides s;
  const int64_t wd[8] = {d, d, dv, dv, dv, d, d, dv};
  int64_t* all[8] = {s.q, s.k, s.v, s.out, s.grad_out, s.grad_q, s.grad_k, s.grad_v};
  for (int t = 0; t < 8; ++t) {
    all[t][0] = H * N * wd[t];
    all[t][1] = N * wd[t];
    all[t][2] = wd[t];
  }
  s.bias[0] = H * N * N; s.bias[1] = N * N; s.bias[2] = N;
  s.lse[0] = H * N; s.lse[1] = N;
  return s;
}

// Groups of 64 rows per (b, h) in the row-statistics workspace.
int64_t bwd_groups(int64_t N) { return (N + fa::kBwdQT - 1) / fa::kBwdQT * 2; }

int check_bwd_shape(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype, int mask) {
  const int st = check_shape(B, H, N, d, dv, dtype, mask);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_DTYPE;
  if (!mfma_width(d) || !mfma_width(dv)) return FA_ERR_SHAPE;
  // rows of the statistics workspace are indexed with 32-bit integers
  if ((B * H) * bwd_groups(N) * 64 >= ((int64_t)1 << 31)) return FA_ERR_SHAPE;
  return FA_OK;
}

// Work plan of the gradients. Without a split, one dK/dV unit per (key tile, b*h) and
// one dQ unit per (query tile, b*h). With few tiles (fewer dK/dV units than CUs), each
// tile's loop (query steps of 64 rows for a key tile, key tiles of 64 for a query tile)
// is cut into chunks of about equal length so that the grid has about 2 units per CU;
// dK/dV steps cost about 4/3 of a dQ step (four products against three), which would
// give the dK/dV kind 4/7 of the units; 9/14 measured about 2% faster on a causal head
// of 8192 (its units also write the larger partials), 5/7 slower again.
struct BwdPlan {
  bool split = false;
  int n_tiles = 0;
  int units_kv = 0, units_q = 0;
  std::vector<uint32_t> unit;  // dK/dV units, then dQ units
  uint8_t nch_kv[fa::kMaxBwdTiles] = {}, nch_q[fa::kMaxBwdTiles] = {};
  size_t stat_bytes = 0, part_kv_floats = 0, part_q_floats = 0, ws_bytes = 0;
};

int64_t bwd_kv_steps(int64_t N, int kt, bool causal) { return (N - (causal ? (int64_t)kt * fa::kBwdKT : 0) + 63) / 64; }
int64_t bwd_q_steps(int64_t N, int qt, bool causal) {
  const int64_t nt = (N + 63) / 64;
  return causal ? std::min<int64_t>(nt, ((int64_t)qt * fa::kBwdQT + fa::kBwdQT - 1) / 64 + 1) : nt;
}

BwdPlan make_bwd_plan(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, bool causal, int cus) {
  BwdPlan pl;
  const int64_t BH = B * H;
  const int64_t nt = (N + fa::kBwdKT - 1) / fa::kBwdKT;
  pl.n_tiles = (int)nt;
  pl.stat_bytes = round_up((size_t)BH * (size_t)bwd_groups(N) * 128 * sizeof(float), 256);
  const int env_units = env_int("FA_BWD_UNITS");
  const int64_t target = std::min<int64_t>(fa::kMaxBwdUnits, env_units > 0 ? env_units : cus * 2);
  pl.split = BH * nt < cus && BH <= 64 && nt <= fa::kMaxBwdTiles && nt > 0 && target >= 2 * BH * nt;
  if (!pl.split) {
    pl.units_kv = pl.units_q = (int)(BH * nt);
    pl.ws_bytes = pl.stat_bytes;
    return pl;
  }
  // chunk lengths: the dK/dV kind gets 9/14 of the target units, dQ the rest
  std::vector<int64_t> skv(nt), sq(nt);
  int64_t tot_kv = 0, tot_q = 0;
  for (int t = 0; t < nt; ++t) {
    skv[t] = bwd_kv_steps(N, t, causal);
    sq[t] = bwd_q_steps(N, t, causal);
    tot_kv += BH * skv[t];
    tot_q += BH * sq[t];
  }
  const int64_t units_kv = target * 9 / 14, units_q = target - units_kv;
  int64_t len_kv = std::max<int64_t>(1, (tot_kv + units_kv - 1) / units_kv);
  int64_t len_q = std::max<int64_t>(1, (tot_q + units_q - 1) / units_q);
  auto count = [&](const std::vector<int64_t>& st, int64_t len) {
    int64_t u = 0;
    for (int t = 0; t < nt; ++t) u += BH * std::min<int64_t>(fa::kMaxBwdChunks, (st[t] + len - 1) / len);
    return u;
  };
  while (count(skv, len_kv) + count(sq, len_q) > fa::kMaxBwdUnits) {
    ++len_kv;
    ++len_q;
  }
  // units: key tiles from the first (longest under a causal mask), query tiles from the
  // last; b*h, then chunks; chunk c of n covers steps [c*s/n, (c+1)*s/n)
  auto emit = [&](const std::vector<int64_t>& st, int64_t len, bool rev, uint8_t* nch) {
    int u0 = (int)pl.unit.size();
    for (int i = 0; i < nt; ++i) {
      const int t = rev ? (int)nt - 1 - i : i;
      const int n = (int)std::min<int64_t>(fa::kMaxBwdChunks, (st[t] + len - 1) / len);
      nch[t] = (uint8_t)n;
      for (int64_t bh = 0; bh < BH; ++bh)
        for (int c = 0; c < n; ++c) {
          const int64_t b0 = c * st[t] / n, b1 = (c + 1) * st[t] / n;
          pl.unit.push_back((uint32_t)t | ((uint32_t)b0 << 8) | ((uint32_t)(b1 - b0) << 17) | ((uint32_t)bh << 26));
        }
    }
    return (int)pl.unit.size() - u0;
  };
  pl.units_kv = emit(skv, len_kv, false, pl.nch_kv);
  pl.units_q = emit(sq, len_q, causal, pl.nch_q);
  pl.part_kv_floats = (size_t)pl.units_kv * fa::kBwdKT * (size_t)(d + dv);
  pl.part_q_floats = (size_t)pl.units_q * fa::kBwdQT * (size_t)d;
  pl.ws_bytes = pl.stat_bytes + round_up((pl.part_kv_floats + pl.part_q_floats) * sizeof(float), 256);
  return pl;
}

std::mutex g_bwd_plan_mu;
std::map<std::array<int64_t, 7>, std::shared_ptr<const BwdPlan>> g_bwd_plans;

std::shared_ptr<const BwdPlan> cached_bwd_plan(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, bool causal,
                                               int cus) {
  const std::array<int64_t, 7> key{B, H, N, d, dv, causal ? 1 : 0, cus};
  std::lock_guard<std::mutex> lk(g_bwd_plan_mu);
  auto it = g_bwd_plans.find(key);
  if (it != g_bwd_plans.end()) return it->second;
  if (g_bwd_plans.size() > 256) g_bwd_plans.clear();
  auto pl = std::make_shared<const BwdPlan>(make_bwd_plan(B, H, N, d, dv, causal, cus));
  g_bwd_plans[key] = pl;
  return pl;
}

int validate_bwd(const BwdProblem& P) {
  int st = check_bwd_shape(P.B, P.H, P.N, P.d, P.dvw, P.dtype, P.mask);
  if (st != FA_OK) return st;
  if (P.B * P.H * P.N == 0) return FA_OK;
  if (!P.q || !P.k || !P.v || !P.out || !P.dout || !P.lse || !P.dq || !P.dk || !P.dv) return FA_ERR_NULL;
  const fa_bwd_strides& s = P.st;
  const void* ptrs[8] = {P.q, P.k, P.v, P.out, P.dout, P.dq, P.dk, P.dv};
  const int64_t* strd[8] = {s.q, s.k, s.v, s.out, s.grad_out, s.grad_q, s.grad_k, s.grad_v};
  const int64_t width[8] = {P.d, P.d, P.dvw, P.dvw, P.dvw, P.d, P.d, P.dvw};
  for (int t = 0; t < 8; ++t)
    for (int i = 0; i < 3; ++i)
      if (strd[t][i] < 0) return FA_ERR_STRIDE;
  for (int i = 0; i < 3; ++i)
    if (s.bias[i] < 0) return FA_ERR_STRIDE;
  if (s.lse[0] < 0 || s.lse[1] < 0) return FA_ERR_STRIDE;
  // tiles of q, k, v and dO are addressed with 32-bit byte offsets
  if (s.q[2] >= kMaxRowStride || s.k[2] >= kMaxRowStride || s.v[2] >= kMaxRowStride ||
      s.grad_out[2] >= kMaxRowStride)
    return FA_ERR_STRIDE;
  const int64_t sz[3] = {P.B, P.H, P.N};
  for (int t = 5; t < 8; ++t)
    if (!non_overlapping(sz, strd[t], 3, width[t])) return FA_ERR_STRIDE;
  for (int t = 0; t < 8; ++t) {
    if (!aligned(ptrs[t], 16)) return FA_ERR_ALIGN;
    for (int i = 0; i < 3; ++i)
      if ((strd[t][i] * 2) % 16 != 0) return FA_ERR_ALIGN;
  }
  if (P.bias && !aligned(P.bias, 4)) return FA_ERR_ALIGN;
  if (!aligned(P.lse, 4)) return FA_ERR_ALIGN;
  // outputs overlap no input and no other output
  Range r[10];
  for (int t = 0; t < 8; ++t) r[t] = extent(ptrs[t], sz, strd[t], 3, width[t], 2);
  r[8] = extent(P.lse, sz, s.lse, 2, P.N, 4);
  r[9] = P.bias ? extent(P.bias, sz, s.bias, 3, P.N, 4) : Range{0, 0};
  for (int o = 5; o < 8; ++o)
    for (int t = 0; t < 10; ++t)
      if (t != o && overlaps(r[o], r[t])) return FA_ERR_ALIAS;
  return FA_OK;
}

BwdProblem make_bwd_problem(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, const float* bias, int mask_mode, void* dq, void* dk, void* dv,
                            int64_t B, int64_t H, int64_t N, int64_t d, int64_t dvw,
                            const fa_bwd_strides* strides, int dtype) {
  BwdProblem P;
  P.q = q; P.k = k; P.v = v; P.out = out; P.dout = dout; P.lse = lse; P.bias = bias;
  P.dq = dq; P.dk = dk; P.dv = dv;
  P.B = B; P.H = H; P.N = N; P.d = d; P.dvw = dvw; P.mask = mask_mode; P.dtype = dtype;
  P.st = strides ? *strides : contiguous_bwd_strides(H, N, d, dvw);
  return P;
}

int run_bwd(const BwdProblem& P, const BwdPlan& pl, void* ws, hipStream_t stream) {
  fa::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  const fa_bwd_strides& s = P.st;
  p.q = P.q; p.k = P.k; p.v = P.v; p.out = P.out; p.dout = P.dout; p.lse = P.lse; p.bias = P.bias;
  p.grad_q = P.dq; p.grad_k = P.dk; p.grad_v = P.dv;
  p.rowstat = static_cast<float*>(ws);
  p.q_sb = s.q[0]; p.q_sh = s.q[1]; p.q_sn = s.q[2];
  p.k_sb = s.k[0]; p.k_sh = s.k[1]; p.k_sn = s.k[2];
  p.v_sb = s.v[0]; p.v_sh = s.v[1]; p.v_sn = s.v[2];
  p.o_sb = s.out[0]; p.o_sh = s.out[1]; p.o_sn = s.out[2];
  p.do_sb = s.grad_out[0]; p.do_sh = s.grad_out[1]; p.do_sn = s.grad_out[2];
  p.dq_sb = s.grad_q[0]; p.dq_sh = s.grad_q[1]; p.dq_sn = s.grad_q[2];
  p.dk_sb = s.grad_k[0]; p.dk_sh = s.grad_k[1]; p.dk_sn = s.grad_k[2];
  p.dv_sb = s.grad_v[0]; p.dv_sh = s.grad_v[1]; p.dv_sn = s.grad_v[2];
  p.b_sb = s.bias[0]; p.b_sh = s.bias[1]; p.b_si = s.bias[2];
  p.l_sb = s.lse[0]; p.l_sh = s.lse[1];
  p.B = (int)P.B; p.H = (int)P.H; p.N = (int)P.N; p.d = (int)P.d; p.dv = (int)P.dvw;
  p.n_grp = (int)bwd_groups(P.N);
  p.bias_vec4 = P.bias && aligned(P.bias, 16) && s.bias[0] % 4 == 0 && s.bias[1] % 4 == 0 && s.bias[2] % 4 == 0;
  p.causal = P.mask == FA_MASK_CAUSAL;
  p.scale = (float)(1.0 / std::sqrt((double)P.d));
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.d));
  p.sqrt_d = (float)std::sqrt((double)P.d);
  p.n_kv_blocks = pl.units_kv;
  p.split = pl.split ? 1 : 0;
  p.n_tiles = pl.n_tiles;
  if (pl.split) {
    p.part = reinterpret_cast<float*>(static_cast<char*>(ws) + pl.stat_bytes);
    p.part_q_off = (int64_t)pl.part_kv_floats;
    std::copy(pl.unit.begin(), pl.unit.end(), p.unit);
    std::copy(pl.nch_kv, pl.nch_kv + fa::kMaxBwdTiles, p.nch_kv);
    std::copy(pl.nch_q, pl.nch_q + fa::kMaxBwdTiles, p.nch_q);
  }
  const hipError_t e = fa::launch_bwd(p, pl.units_kv + pl.units_q, P.dtype == FA_F16, stream);
  if (env_int("FA_LOG"))
    std::fprintf(stderr, "[fa] bwd B=%lld H=%lld N=%lld d=%lld dv=%lld causal=%d bias=%d split=%d units=%d+%d ws=%zu\n",
                 (long long)P.B, (long long)P.H, (long long)P.N, (long long)P.d, (long long)P.dvw, p.causal,
                 P.bias != nullptr, p.split, pl.units_kv, pl.units_q, pl.ws_bytes);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd_qk_ex(const void* q, const void* k, const void* v, const float* bias, int mask_mode, void* out,
                 float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                 const fa_strides* strides, int dtype, void* stream, void* workspace, size_t workspace_bytes) {
  const Problem P = make_problem(q, k, v, bias, mask_mode, out, lse, B, H, Nq, Nk, d, dv, strides, dtype);
  int st = validate(P);
  if (st != FA_OK) return st;
  if (B * H * Nq == 0) return FA_OK;
  int dev = 0;
  DevInfo di;
  if ((st = device_info(&dev, &di)) != FA_OK) return st;
  const std::shared_ptr<const Plan> plan = cached_plan(B, H, Nq, Nk, d, dv, dtype, mask_mode, di.cus);
  const Plan& pl = *plan;
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes || !aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  }
  return run(P, pl, workspace, static_cast<hipStream_t>(stream));
}

int fa_fwd_qk(const void* q, const void* k, const void* v, const float* bias, int mask_mode, void* out,
              float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
              const fa_strides* strides, int dtype, void* stream) {
  const Problem P = make_problem(q, k, v, bias, mask_mode, out, lse, B, H, Nq, Nk, d, dv, strides, dtype);
  int st = validate(P);
  if (st != FA_OK) return st;
  if (B * H * Nq == 0) return FA_OK;
  int dev = 0;
  DevInfo di;
  if ((st = device_info(&dev, &di)) != FA_OK) return st;
  const std::shared_ptr<const Plan> plan = cached_plan(B, H, Nq, Nk, d, dv, dtype, mask_mode, di.cus);
  const Plan& pl = *plan;
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = owned_workspace(dev, static_cast<hipStream_t>(stream), pl.ws_bytes, &ws);
    if (st != FA_OK) return st;
  }
  return run(P, pl, ws, static_cast<hipStream_t>(stream));
}

int fa_fwd_qk_noalloc(const void* q, const void* k, const void* v, const float* bias, int mask_mode, void* out,
                      float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                      const fa_strides* strides, int dtype, void* stream) {
  const Problem P = make_problem(q, k, v, bias, mask_mode, out, lse, B, H, Nq, Nk, d, dv, strides, dtype);
  int st = validate(P);
  if (st != FA_OK) return st;
  if (B * H * Nq == 0) return FA_OK;
  int dev = 0;
  DevInfo di;
  if ((st = device_info(&dev, &di)) != FA_OK) return st;
  const std::shared_ptr<const Plan> plan = cached_plan(B, H, Nq, Nk, d, dv, dtype, mask_mode, di.cus);
  const Plan& pl = *plan;
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    if (pl.ws_bytes > kStaticScratchBytes) return FA_ERR_WORKSPACE;
    if ((st = static_scratch(dev, &ws)) != FA_OK) return st;
  }
  return run(P, pl, ws, static_cast<hipStream_t>(stream));
}

size_t fa_fwd_qk_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, int dtype,
                                int mask_mode) {
  if (check_shape_qk(B, H, Nq, Nk, d, dv, dtype, mask_mode) != FA_OK) return 0;
  if (B * H * Nq == 0) return 0;
  int dev = 0;
  DevInfo di;
  if (device_info(&dev, &di) != FA_OK) return 0;
  return cached_plan(B, H, Nq, Nk, d, dv, dtype, mask_mode, di.cus)->ws_bytes;
}

int fa_fwd_ex(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
              void* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
              const fa_strides* strides, int dtype, void* stream, void* workspace,
              size_t workspace_bytes) {
  return fa_fwd_qk_ex(q, k, v, bias, mask_mode, out, lse, B, H, N, N, d, dv, strides, dtype, stream, workspace,
                      workspace_bytes);
}

int fa_fwd(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
           void* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
           const fa_strides* strides, int dtype, void* stream) {
  return fa_fwd_qk(q, k, v, bias, mask_mode, out, lse, B, H, N, N, d, dv, strides, dtype, stream);
}

size_t fa_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype,
                             int mask_mode) {
  return fa_fwd_qk_workspace_size(B, H, N, N, d, dv, dtype, mask_mode);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "unsupported or invalid shape (d and dv: 1..256; gradients: 64 or 128)";
    case FA_ERR_DTYPE: return "unsupported dtype";
    case FA_ERR_MASK: return "unsupported mask mode";
    case FA_ERR_STRIDE: return "negative stride or overlapping output rows";
    case FA_ERR_ALIGN: return "misaligned pointer";
    case FA_ERR_ALIAS: return "an output overlaps an input or the other output";
    case FA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case FA_ERR_ALLOC: return "workspace allocation failed";
    default: return "unknown status";
  }
}

int fa_version(void) { return FA_VERSION; }

int fa_plan_describe_qk(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, int dtype,
                        int mask_mode, int compute_units, fa_plan_info* info, uint32_t* unit_info,
                        int max_units) {
  if (!info || compute_units < 1) return FA_ERR_NULL;
  const int st = check_shape_qk(B, H, Nq, Nk, d, dv, dtype, mask_mode);
  if (st != FA_OK) return st;
  const std::shared_ptr<const Plan> plan = cached_plan(B, H, Nq, Nk, d, dv, dtype, mask_mode, compute_units);
  const Plan& pl = *plan;
  info->split = pl.split ? 1 : 0;
  info->n_qtiles = pl.mfma ? pl.n_qt : 0;
  info->qtile_rows = pl.mfma ? fa::kMfmaBM : fa::kGenericBM;
  info->key_tile = fa::kMfmaBN;
  info->units = pl.mfma ? pl.grid : 0;
  info->merge_blocks = pl.merge_blocks;
  info->workspace_bytes = pl.ws_bytes;
  info->unit_tile_shift = pl.shift;
  if (pl.split && unit_info) {
    int u = 0;
    for (int qt = pl.n_qt - 1; qt >= 0; --qt) {
      const Plan::Ranges& r = pl.ranges[qt];
      for (int64_t bh = 0; bh < B * H; ++bh)
        for (int c = 0; c < r.nch; ++c, ++u)
          if (u < max_units) unit_info[u] = pack_unit(qt, r.begin[c], r.len[c], bh, pl.n_qt == 1, pl.shift);
    }
  }
  return FA_OK;
}

int fa_plan_describe(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype, int mask_mode,
                     int compute_units, fa_plan_info* info, uint32_t* unit_info, int max_units) {
  return fa_plan_describe_qk(B, H, N, N, d, dv, dtype, mask_mode, compute_units, info, unit_info, max_units);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* out, const float* lse,
              const void* grad_out, const float* bias, int mask_mode, void* grad_q, void* grad_k,
              void* grad_v, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
              const fa_bwd_strides* strides, int dtype, void* stream, void* workspace,
              size_t workspace_bytes) {
  const BwdProblem P = make_bwd_problem(q, k, v, out, lse, grad_out, bias, mask_mode, grad_q, grad_k, grad_v,
                                        B, H, N, d, dv, strides, dtype);
  int st = validate_bwd(P);
  if (st != FA_OK) return st;
  if (B * H * N == 0) return FA_OK;
  int dev = 0;
  DevInfo di;
  if ((st = device_info(&dev, &di)) != FA_OK) return st;
  const std::shared_ptr<const BwdPlan> plan = cached_bwd_plan(B, H, N, d, dv, mask_mode == FA_MASK_CAUSAL, di.cus);
  if (!workspace || workspace_bytes < plan->ws_bytes || !aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  return run_bwd(P, *plan, workspace, static_cast<hipStream_t>(stream));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
           const void* grad_out, const float* bias, int mask_mode, void* grad_q, void* grad_k,
           void* grad_v, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
           const fa_bwd_strides* strides, int dtype, void* stream) {
  const BwdProblem P = make_bwd_problem(q, k, v, out, lse, grad_out, bias, mask_mode, grad_q, grad_k, grad_v,
                                        B, H, N, d, dv, strides, dtype);
  int st = validate_bwd(P);
  if (st != FA_OK) return st;
  if (B * H * N == 0) return FA_OK;
  int dev = 0;
  DevInfo di;
  if ((st = device_info(&dev, &di)) != FA_OK) return st;
  const std::shared_ptr<const BwdPlan> plan = cached_bwd_plan(B, H, N, d, dv, mask_mode == FA_MASK_CAUSAL, di.cus);
  void* ws = nullptr;
  st = owned_workspace(dev, static_cast<hipStream_t>(stream), plan->ws_bytes, &ws);
  if (st != FA_OK) return st;
  return run_bwd(P, *plan, ws, static_cast<hipStream_t>(stream));
}

size_t fa_bwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype,
                             int mask_mode) {
  if (check_bwd_shape(B, H, N, d, dv, dtype, mask_mode) != FA_OK) return 0;
  if (B * H * N == 0) return 0;
  int dev = 0;
  DevInfo di;
  if (device_info(&dev, &di) != FA_OK) return 0;
  return cached_bwd_plan(B, H, N, d, dv, mask_mode == FA_MASK_CAUSAL, di.cus)->ws_bytes;
}

void fa_shutdown(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  auto release = [](int dev, void* ptr) {
    (void)hipSetDevice(dev);
    (void)hipDeviceSynchronize();
    (void)hipFree(ptr);
  };
  for (auto& kv : g_ws)
    if (kv.second.ptr) release(kv.first.first, kv.second.ptr);
  for (auto& r : g_ws_retired) release(r.first, r.second);
  g_ws.clear();
  g_ws_retired.clear();
  (void)hipSetDevice(cur);
}

}  // extern "C"

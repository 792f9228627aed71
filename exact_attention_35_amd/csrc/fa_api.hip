// Host side of the C ABI declared in include/fa.h: argument validation, the work
// plan (query tiles and key splits), scratch workspaces, and kernel dispatch.
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
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "fa.h"
#include "fa_internal.h"

namespace {

using fa::Params;

constexpr int kMaxSplitTiles = 255;           // (b, h, query tile)s eligible for a split (8-bit fields)
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
  int64_t B, H, N, d, dv;
  int mask, dtype;
  fa_strides st;
};

fa_strides contiguous_strides(int64_t H, int64_t N, int64_t d, int64_t dv) {
  fa_strides s;
  s.q[0] = H * N * d; s.q[1] = N * d; s.q[2] = d;
  s.k[0] = H * N * d; s.k[1] = N * d; s.k[2] = d;
  s.v[0] = H * N * dv; s.v[1] = N * dv; s.v[2] = dv;
  s.out[0] = H * N * dv; s.out[1] = N * dv; s.out[2] = dv;
  s.bias[0] = H * N * N; s.bias[1] = N * N; s.bias[2] = N;
  s.lse[0] = H * N; s.lse[1] = N;
  return s;
}

bool supported_width(int64_t x) { return x == 64 || x == 128; }

// Size/shape/dtype/mask checks shared by the size query and the forward calls.
int check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype, int mask) {
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (mask != FA_MASK_NONE && mask != FA_MASK_CAUSAL) return FA_ERR_MASK;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (!supported_width(d) || !supported_width(dv)) return FA_ERR_SHAPE;
  const int64_t lim = (int64_t)1 << 30;
  if (B > lim || H > lim || N > lim) return FA_ERR_SHAPE;
  if (B * H > lim || (B * H) * ((N + 63) / 64) > lim) return FA_ERR_SHAPE;
  return FA_OK;
}

int validate(const Problem& P) {
  int st = check_shape(P.B, P.H, P.N, P.d, P.dv, P.dtype, P.mask);
  if (st != FA_OK) return st;
  if (P.B * P.H * P.N == 0) return FA_OK;
  if (!P.q || !P.k || !P.v || !P.out) return FA_ERR_NULL;
  const fa_strides& s = P.st;
  const int64_t* all[] = {s.q, s.k, s.v, s.out, s.bias};
  for (int t = 0; t < 5; ++t)
    for (int i = 0; i < 3; ++i)
      if (all[t][i] < 0) return FA_ERR_STRIDE;
  if (s.lse[0] < 0 || s.lse[1] < 0) return FA_ERR_STRIDE;
  // the bf16 kernel addresses a 64-row key tile with 32-bit byte offsets
  if (P.dtype == FA_BF16 && (s.k[2] >= kMaxRowStride || s.v[2] >= kMaxRowStride)) return FA_ERR_STRIDE;
  const int64_t sz[3] = {P.B, P.H, P.N};
  if (!non_overlapping(sz, s.out, 3, P.dv)) return FA_ERR_STRIDE;
  if (P.lse && !non_overlapping(sz, s.lse, 2, P.N)) return FA_ERR_STRIDE;

  const int es = P.dtype == FA_BF16 ? 2 : 4;
  const void* ptrs[4] = {P.q, P.k, P.v, P.out};
  const int64_t* strd[4] = {s.q, s.k, s.v, s.out};
  for (int t = 0; t < 4; ++t) {
    if (!aligned(ptrs[t], 16)) return FA_ERR_ALIGN;
    for (int i = 0; i < 3; ++i)
      if ((strd[t][i] * es) % 16 != 0) return FA_ERR_ALIGN;
  }
  if (P.bias && !aligned(P.bias, 4)) return FA_ERR_ALIGN;
  if (P.lse && !aligned(P.lse, 4)) return FA_ERR_ALIGN;

  // aliasing: outputs must not overlap inputs or each other
  const Range rq = extent(P.q, sz, s.q, 3, P.d, es);
  const Range rk = extent(P.k, sz, s.k, 3, P.d, es);
  const Range rv = extent(P.v, sz, s.v, 3, P.dv, es);
  const Range ro = extent(P.out, sz, s.out, 3, P.dv, es);
  if (overlaps(ro, rq) || overlaps(ro, rk) || overlaps(ro, rv)) return FA_ERR_ALIAS;
  Range rb{0, 0};
  if (P.bias) {
    const int64_t bsz[3] = {P.B, P.H, P.N};
    rb = extent(P.bias, bsz, s.bias, 3, P.N, 4);
    if (overlaps(ro, rb)) return FA_ERR_ALIAS;
  }
  if (P.lse) {
    const Range rl = extent(P.lse, sz, s.lse, 2, P.N, 4);
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
  int chunk_tiles = 0;  // 0: no split over keys
  int grid = 0;         // forward workgroups (units)
  int merge_grid = 0;   // merge workgroups (0: no merge kernel)
  size_t ws_bytes = 0;
  size_t off_ml = 0, off_o = 0;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int env_int(const char* name) {
  const char* e = std::getenv(name);
  return e ? std::atoi(e) : 0;
}

// Key tiles of query tile qt (causal tiles stop at the diagonal).
int64_t qtile_ntiles(int64_t N, int qt, bool causal) {
  const int64_t bm = fa::kMfmaBM, bn = fa::kMfmaBN;
  const int64_t kv = causal ? std::min(N, (qt + 1) * bm) : N;
  return (kv + bn - 1) / bn;
}

Plan make_plan(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype, int mask, int cus) {
  Plan pl;
  pl.mfma = dtype == FA_BF16;  // d, dv in {64, 128} already checked
  if (!pl.mfma) return pl;
  const bool causal = mask == FA_MASK_CAUSAL;
  const int bm = fa::kMfmaBM;
  pl.n_qt = (int)((N + bm - 1) / bm);
  const int64_t BH = B * H;
  const int64_t tiles = BH * pl.n_qt;
  pl.grid = (int)tiles;
  if (tiles <= 0 || tiles >= cus || tiles > kMaxSplitTiles || pl.n_qt > fa::kMaxSplitQTiles) return pl;
  // Too few query tiles to occupy the chip: cut each tile's key range into ranges
  // of about `chunk` key tiles, so that about `target` ranges (two workgroups per CU)
  // exist in total.
  int64_t total = 0;
  for (int qt = 0; qt < pl.n_qt; ++qt) total += BH * qtile_ntiles(N, qt, causal);
  const int64_t target = std::min<int64_t>(fa::kMaxSplitUnits,
                                           env_int("FA_SPLIT_UNITS") > 0 ? env_int("FA_SPLIT_UNITS") : 2 * (int64_t)cus);
  int64_t chunk = std::max<int64_t>(1, (total + target - 1) / target);
  // no query tile may be cut into more than kMaxRanges ranges
  const int64_t nt_max = qtile_ntiles(N, pl.n_qt - 1, causal);
  chunk = std::max<int64_t>(chunk, (nt_max + fa::kMaxRanges - 1) / fa::kMaxRanges);
  // the ranges must fit in one wave of workgroups: grow the chunk until they do
  int64_t units = 0;
  bool any_split = false;
  for (;; ++chunk) {
    units = 0;
    any_split = false;
    for (int qt = 0; qt < pl.n_qt; ++qt) {
      const int64_t nch = (qtile_ntiles(N, qt, causal) + chunk - 1) / chunk;
      units += BH * nch;
      any_split |= nch > 1;
    }
    if (units <= target || !any_split) break;
  }
  if (!any_split) return pl;
  pl.chunk_tiles = (int)chunk;
  pl.grid = (int)units;
  pl.merge_grid = (int)(tiles * (fa::kMergeGroups * dv / 128));
  pl.off_ml = 0;
  pl.off_o = round_up(units * 2 * bm * sizeof(float), 256);
  pl.ws_bytes = round_up(pl.off_o + (size_t)units * bm * dv * sizeof(float), 256);
  return pl;
}

// ---------------------------------------------------------------- launch
int run(const Problem& P, const Plan& pl, void* ws, hipStream_t stream) {
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
  p.causal = P.mask == FA_MASK_CAUSAL;
  p.bias_vec4 = P.bias && aligned(P.bias, 16) && s.bias[0] % 4 == 0 && s.bias[1] % 4 == 0 && s.bias[2] % 4 == 0;
  p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)P.d));
  p.scale = (float)(1.0 / std::sqrt((double)P.d));
  p.n_qt = pl.n_qt;
  p.chunk_tiles = pl.chunk_tiles;
  if (pl.chunk_tiles > 0) {  // unit table of the split plan (query tiles from the last)
    int32_t acc = 0;
    for (int qt = pl.n_qt - 1; qt >= 0; --qt) {
      const int64_t nch = (qtile_ntiles(P.N, qt, p.causal) + pl.chunk_tiles - 1) / pl.chunk_tiles;
      p.ubase[qt] = acc;
      p.nchq[qt] = (uint8_t)nch;
      for (int64_t bh = 0; bh < P.B * P.H; ++bh)
        for (int c = 0; c < nch; ++c)
          p.unit_info[acc + bh * nch + c] =
              (uint32_t)qt | (uint32_t)bh << 8 | (uint32_t)c << 16 | (uint32_t)nch << 24;
      acc += (int32_t)(P.B * P.H * nch);
    }
    p.ubase[pl.n_qt] = acc;
  }
  if (pl.ws_bytes > 0) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    p.part_ml = reinterpret_cast<float*>(w + pl.off_ml);
    p.part_o = reinterpret_cast<float*>(w + pl.off_o);
  }
  hipError_t e = pl.mfma ? fa::launch_mfma_bf16(p, pl.grid, pl.merge_grid > 0, stream)
                         : fa::launch_generic(p, P.dtype == FA_BF16, stream);
  if (std::getenv("FA_LOG"))
    std::fprintf(stderr, "[fa] %s B=%lld H=%lld N=%lld d=%lld dv=%lld causal=%d bias=%d n_qt=%d chunk=%d grid=%d merge=%d ws=%zu\n",
                 pl.mfma ? "mfma_bf16" : (P.dtype == FA_BF16 ? "generic_bf16" : "generic_f32"),
                 (long long)P.B, (long long)P.H, (long long)P.N, (long long)P.d, (long long)P.dv,
                 p.causal, P.bias != nullptr, pl.n_qt, pl.chunk_tiles, pl.grid, pl.merge_grid, pl.ws_bytes);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

Problem make_problem(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
                     void* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
                     const fa_strides* strides, int dtype) {
  Problem P;
  P.q = q; P.k = k; P.v = v; P.bias = bias; P.out = out; P.lse = lse;
  P.B = B; P.H = H; P.N = N; P.d = d; P.dv = dv; P.mask = mask_mode; P.dtype = dtype;
  P.st = strides ? *strides : contiguous_strides(H, N, d, dv);
  return P;
}

// ---------------------------------------------------------------- owned workspaces
struct OwnedWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, OwnedWs> g_ws;

int owned_workspace(int dev, hipStream_t stream, size_t need, void** out) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  OwnedWs& w = g_ws[{dev, stream}];
  if (w.bytes < need) {
    if (w.ptr) {
      if (hipStreamSynchronize(stream) != hipSuccess) return FA_ERR_ALLOC;
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, need) != hipSuccess) return FA_ERR_ALLOC;
    w.ptr = p;
    w.bytes = need;
  }
  *out = w.ptr;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_ex(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
              void* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
              const fa_strides* strides, int dtype, void* stream, void* workspace,
              size_t workspace_bytes) {
  const Problem P = make_problem(q, k, v, bias, mask_mode, out, lse, B, H, N, d, dv, strides, dtype);
  int st = validate(P);
  if (st != FA_OK) return st;
  if (B * H * N == 0) return FA_OK;
  int dev = 0;
  DevInfo di;
  if ((st = device_info(&dev, &di)) != FA_OK) return st;
  const Plan pl = make_plan(B, H, N, d, dv, dtype, mask_mode, di.cus);
  if (pl.ws_bytes > 0) {
    if (!workspace || workspace_bytes < pl.ws_bytes || !aligned(workspace, 256)) return FA_ERR_WORKSPACE;
  }
  return run(P, pl, workspace, static_cast<hipStream_t>(stream));
}

int fa_fwd(const void* q, const void* k, const void* v, const float* bias, int mask_mode,
           void* out, float* lse, int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv,
           const fa_strides* strides, int dtype, void* stream) {
  const Problem P = make_problem(q, k, v, bias, mask_mode, out, lse, B, H, N, d, dv, strides, dtype);
  int st = validate(P);
  if (st != FA_OK) return st;
  if (B * H * N == 0) return FA_OK;
  int dev = 0;
  DevInfo di;
  if ((st = device_info(&dev, &di)) != FA_OK) return st;
  const Plan pl = make_plan(B, H, N, d, dv, dtype, mask_mode, di.cus);
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    st = owned_workspace(dev, static_cast<hipStream_t>(stream), pl.ws_bytes, &ws);
    if (st != FA_OK) return st;
  }
  return run(P, pl, ws, static_cast<hipStream_t>(stream));
}

size_t fa_fwd_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d, int64_t dv, int dtype,
                             int mask_mode) {
  if (check_shape(B, H, N, d, dv, dtype, mask_mode) != FA_OK) return 0;
  if (B * H * N == 0) return 0;
  int dev = 0;
  DevInfo di;
  if (device_info(&dev, &di) != FA_OK) return 0;
  return make_plan(B, H, N, d, dv, dtype, mask_mode, di.cus).ws_bytes;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "unsupported or invalid shape (d and dv must be 64 or 128)";
    case FA_ERR_DTYPE: return "unsupported dtype";
    case FA_ERR_MASK: return "unsupported mask mode";
    case FA_ERR_STRIDE: return "negative stride or overlapping output rows";
    case FA_ERR_ALIGN: return "misaligned pointer or stride";
    case FA_ERR_ALIAS: return "an output overlaps an input or the other output";
    case FA_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case FA_ERR_ALLOC: return "workspace allocation failed";
    default: return "unknown status";
  }
}

int fa_version(void) { return FA_VERSION; }

void fa_shutdown(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (auto& kv : g_ws) {
    if (kv.second.ptr) {
      int cur = 0;
      (void)hipGetDevice(&cur);
      (void)hipSetDevice(kv.first.first);
      (void)hipDeviceSynchronize();
      (void)hipFree(kv.second.ptr);
      (void)hipSetDevice(cur);
    }
  }
  g_ws.clear();
}

}  // extern "C"

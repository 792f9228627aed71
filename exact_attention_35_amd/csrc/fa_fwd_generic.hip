// General attention-forward kernel on the vector ALUs (fp32, bf16 and fp16 inputs).
//
// It applies the online-softmax recurrence of the page "编译器与内核" (Compilers and
// kernels), section "FlashAttention 围绕 IO 改写算法", one key block at a time: a
// workgroup owns 64 query rows; each key block of 32 keys is staged in LDS (converted
// to fp32), the 32 scores of a row are formed, then the block max b_t, the new
// running max m_t, the rescale alpha_t = exp(m_{t-1} - m_t), the normaliser l_t and the
// numerator o_t are updated, and O_i = o_T / l_T is written at the end.
//
// Exponentials are taken in base 2: scores are carried as S * log2(e) (the factor is
// folded into the 1/sqrt(d) scale, and the bias is multiplied by log2(e)), so
// exp(S - m) = exp2(S*log2e - m*log2e). The hardware v_exp_f32 / v_log_f32
// instructions supply exp2 and log2.
//
// Four lanes share one query row: lane `sub` owns the dims sub, sub+4, sub+8, ... of
// q and of o, so the four lanes of a row read consecutive LDS words (no bank
// conflict) and every row of the workgroup reads the same key (an LDS broadcast).
// This kernel is the general path: fp32, fp16, any width up to 256, and any element-
// aligned layout; the bf16 fast path (widths 64 and 128, 16-byte aligned rows) runs on
// the matrix cores (fa_fwd_mfma.hip).

#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }  // exact for every T here
template <typename T>
__device__ __forceinline__ T from_f32(float x) { return (T)x; }    // round to nearest even

// D, DV: the widths rounded up to 32, 64, 128 or 256; the actual widths p.d, p.dv mask
// the loads (dims past them read as 0, which adds nothing to a dot product) and the
// stores.
// BM: query rows per workgroup (4 lanes each, so BM * 4 threads); BK: keys per block.
template <typename T, int D, int DV, int BM = kGenericBM, int BK = 32>
__global__ __launch_bounds__(BM * 4) void fwd_generic(Params p) {
  constexpr int NT = BM * 4;      // threads
  constexpr int LPR = 4;          // lanes per query row
  constexpr int DQ = D / LPR;
  constexpr int DO = DV / LPR;
  __shared__ float Ks[BK][D];
  __shared__ float Vs[BK][DV];
  const int d = p.d, dv = p.dv;

  const int tid = threadIdx.x;
  const int row = tid / LPR;
  const int sub = tid % LPR;
  // 1-D grid: block = (b*h) * n_qt + query tile
  const int n_qt = (p.Nq + BM - 1) / BM;
  const int bh = blockIdx.x / n_qt;
  const int b = bh / p.H;
  const int h = bh % p.H;
  const int q0 = (blockIdx.x % n_qt) * BM;
  const int qi = q0 + row;
  const bool qvalid = qi < p.Nq;

  const T* qp = static_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* kp = static_cast<const T*>(p.k) + b * p.k_sb + h * p.k_sh;
  const T* vp = static_cast<const T*>(p.v) + b * p.v_sb + h * p.v_sh;
  const float* bp = p.bias ? p.bias + b * p.b_sb + h * p.b_sh + (int64_t)(qvalid ? qi : 0) * p.b_si
                           : nullptr;

  float qr[DQ];
#pragma unroll
  for (int i = 0; i < DQ; ++i)
    qr[i] = qvalid && sub + LPR * i < d ? to_f32<T>(qp[(int64_t)qi * p.q_sn + sub + LPR * i]) : 0.f;

  float o[DO];
#pragma unroll
  for (int i = 0; i < DO; ++i) o[i] = 0.f;
  float m = -INFINITY;  // running max, base-2 units
  float l = 0.f;        // running normaliser

  // causal: key j is allowed for row i iff j <= i + coff
  const int kv_end = p.causal ? min(p.N, max(q0 + BM + p.coff, 0)) : p.N;
  for (int kv0 = 0; kv0 < kv_end; kv0 += BK) {
    __syncthreads();  // previous block fully consumed
    for (int idx = tid; idx < BK * D; idx += NT) {
      const int r = idx / D, c = idx % D;
      const int key = kv0 + r;
      Ks[r][c] = key < p.N && c < d ? to_f32<T>(kp[(int64_t)key * p.k_sn + c]) : 0.f;
    }
    for (int idx = tid; idx < BK * DV; idx += NT) {
      const int r = idx / DV, c = idx % DV;
      const int key = kv0 + r;
      Vs[r][c] = key < p.N && c < dv ? to_f32<T>(vp[(int64_t)key * p.v_sn + c]) : 0.f;
    }
    __syncthreads();

    // scores of this block (base 2) and the block max b_t
    float s[BK];
    float bmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) acc = fmaf(qr[i], Ks[j][sub + LPR * i], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      const int key = kv0 + j;
      float x = acc * p.scale_log2;
      if (bp && key < p.N && qvalid) x = fmaf(bp[key], kLog2e, x);
      if (key >= p.N || (p.causal && key > qi + p.coff)) x = -INFINITY;
      s[j] = x;
      bmax = fmaxf(bmax, x);
    }
    // m_t = max(m_{t-1}, b_t); while no allowed key has been seen (m_t = -inf) the
    // block adds nothing: using 0 as the reference keeps exp2 away from -inf - -inf.
    const float m_new = fmaxf(m, bmax);
    const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_ref);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < BK; ++j) {
      s[j] = __builtin_amdgcn_exp2f(s[j] - m_ref);
      psum += s[j];
    }
    l = alpha * l + psum;
#pragma unroll
    for (int i = 0; i < DO; ++i) {
      float acc = alpha * o[i];
#pragma unroll
      for (int j = 0; j < BK; ++j) acc = fmaf(s[j], Vs[j][sub + LPR * i], acc);
      o[i] = acc;
    }
    m = m_new;
  }

  if (!qvalid) return;
  T* op = static_cast<T*>(p.out) + b * p.o_sb + h * p.o_sh + (int64_t)qi * p.o_sn;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < DO; ++i)
    if (sub + LPR * i < dv) op[sub + LPR * i] = from_f32<T>(o[i] * inv);
  if (p.lse && sub == 0) {
    p.lse[b * p.l_sb + h * p.l_sh + qi] =
        l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
  }
}

// the width bin of x (1 .. 256): 32, 64, 128 or 256
inline int width_bin(int x) { return x <= 32 ? 32 : x <= 64 ? 64 : x <= 128 ? 128 : 256; }

template <typename T, int D>
hipError_t launch_dv(const Params& p, dim3 grid, hipStream_t stream) {
  switch (width_bin(p.dv)) {
    case 32: FA_LAUNCH_MAIN((fwd_generic<T, D, 32>), grid, dim3(256), stream, p); break;
    case 64: FA_LAUNCH_MAIN((fwd_generic<T, D, 64>), grid, dim3(256), stream, p); break;
    case 128: FA_LAUNCH_MAIN((fwd_generic<T, D, 128>), grid, dim3(256), stream, p); break;
    default: FA_LAUNCH_MAIN((fwd_generic<T, D, 256>), grid, dim3(256), stream, p); break;
  }
  return hipGetLastError();
}

// Other tile shapes (BM, BK) of the fp32 kernel at widths up to 64 and 128, for the
// tile-shape experiment: p.gtile 1: (32, 32), 2: (64, 16), 3: (64, 64), 4: (128, 32).
template <int D, int DV>
hipError_t launch_tile(const Params& p, hipStream_t stream) {
  auto grid = [&](int bm) { return dim3((unsigned)(((p.Nq + bm - 1) / bm) * (int64_t)p.B * p.H)); };
  switch (p.gtile) {
    case 1: FA_LAUNCH_MAIN((fwd_generic<float, D, DV, 32, 32>), grid(32), dim3(128), stream, p); break;
    case 2: FA_LAUNCH_MAIN((fwd_generic<float, D, DV, 64, 16>), grid(64), dim3(256), stream, p); break;
    case 3: FA_LAUNCH_MAIN((fwd_generic<float, D, DV, 64, 64>), grid(64), dim3(256), stream, p); break;
    default: FA_LAUNCH_MAIN((fwd_generic<float, D, DV, 128, 32>), grid(128), dim3(512), stream, p); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const Params& p, hipStream_t stream) {
  if (p.d < 1 || p.d > 256 || p.dv < 1 || p.dv > 256) return hipErrorInvalidValue;
  if constexpr (std::is_same<T, float>::value) {
    if (p.gtile >= 1 && p.gtile <= 4 && p.d <= 128 && p.dv <= 128) {
      const int bd = width_bin(p.d) <= 64 ? 64 : 128, bdv = width_bin(p.dv) <= 64 ? 64 : 128;
      if (bd == 64 && bdv == 64) return launch_tile<64, 64>(p, stream);
      if (bd == 64) return launch_tile<64, 128>(p, stream);
      if (bdv == 64) return launch_tile<128, 64>(p, stream);
      return launch_tile<128, 128>(p, stream);
    }
  }
  const dim3 grid((unsigned)(((p.Nq + kGenericBM - 1) / kGenericBM) * (int64_t)p.B * p.H));
  switch (width_bin(p.d)) {
    case 32: return launch_dv<T, 32>(p, grid, stream);
    case 64: return launch_dv<T, 64>(p, grid, stream);
    case 128: return launch_dv<T, 128>(p, grid, stream);
    default: return launch_dv<T, 256>(p, grid, stream);
  }
}

}  // namespace

hipError_t launch_generic(const Params& p, int dtype, hipStream_t stream) {
  switch (dtype) {
    case 1: return launch_t<__bf16>(p, stream);
    case 2: return launch_t<_Float16>(p, stream);
    default: return launch_t<float>(p, stream);
  }
}

}  // namespace fa

// Measurement probes for the roofline of the attention kernels (include/fa_probe.h).
//
// The page "编译器与内核" (Compilers and kernels), section "屋顶线是上界，不是秒表", bounds a
// kernel by min(P_max, B_max * I) and asks for P_max on the same dtype and instruction
// path as the kernel's FLOP count, and for B_max as the bandwidth the access pattern
// actually reaches, measured rather than copied from a specification sheet. These two
// kernels measure both ceilings on the device at hand:
//  * copy: a streaming copy with 16-byte loads and stores (the widest per-lane global
//    access of gfx950), grid-stride, over buffers much larger than the 256 MB
//    last-level cache, so every byte crosses the HBM boundary once each way;
//  * mfma: back-to-back v_mfma_f32_32x32x16_bf16 (the instruction the attention kernel
//    spends its FLOPs on), four independent accumulator chains per wave and two waves
//    per SIMD, as the attention kernel runs, with no memory traffic in the loop.
// The same page asks for repetitions, quantiles and cold against warm runs. The launch
// timer below gives each main-kernel launch its own pair of events stamped by the kernel's
// dispatch itself, so one launch's time excludes the queue gap that a pair of events
// recorded around the launch would add.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <vector>

#include "fa_internal.h"
#include "fa_mfma_common.h"
#include "fa_probe.h"

namespace {

// Each thread keeps four 16-byte loads in flight before it stores them (one load at a time
// leaves the memory system idle between round trips).
__global__ __launch_bounds__(256) void copy_probe(const fa::u32x4* __restrict__ src,
                                                  fa::u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const fa::u32x4 a = __builtin_nontemporal_load(src + i);
    const fa::u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const fa::u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const fa::u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// Each thread keeps four 16-byte loads in flight and folds them into one word, which each
// workgroup stores once (so the loads are not removed): a read-only stream.
__global__ __launch_bounds__(256) void read_probe(const fa::u32x4* __restrict__ src, int64_t n16,
                                                  unsigned* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  fa::u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const fa::u32x4 a = __builtin_nontemporal_load(src + i);
    const fa::u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const fa::u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const fa::u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  const unsigned w = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  const unsigned any = (unsigned)__builtin_amdgcn_ballot_w64(w != 0u);  // one word per block
  if (threadIdx.x == 0) sink[blockIdx.x] = any;
}

// Issue probe: how the matrix core and the vector ALU of one SIMD share a wave's and two
// waves' instruction streams. MFMA waves run two alternating accumulator chains of
// v_mfma_f32_32x32x16_bf16 and, after each MFMA, K independent v_fma_f32 and E independent
// v_exp_f32 (written in asm so the compiler keeps exactly these); VALU waves run steps of
// 12 independent v_fma_f32 (or 4 v_exp_f32 with E > 0). Each wave times its loop with
// s_memtime (the shader clock) and s_memrealtime (100 MHz, to convert).
// ROLE 0: every wave of a 4-wave block (one per SIMD) is an MFMA wave; ROLE 1: 8-wave
// blocks, waves 0-3 MFMA and 4-7 VALU (waves w and w + 4 share a SIMD); ROLE 2: the same
// blocks with only the MFMA waves working; ROLE 3: only the VALU waves; ROLE 4: all eight
// are VALU waves (two per SIMD).
template <int ROLE, int K, int E>
__global__ __launch_bounds__(512) void issue_probe(float* __restrict__ out, long long* __restrict__ ticks,
                                                   int iters) {
  using fa::bf16x8;
  using fa::floatx16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool mfma_wave = ROLE == 0 || ((ROLE == 1 || ROLE == 2) && wave < 4);
  const bool valu_wave = (ROLE == 1 || ROLE == 3) ? wave >= 4 : ROLE == 4;
  float acc = 0.f;
  long long t = 0, r = 0;
  if (mfma_wave) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.001f * (float)(lane + e));
      b[e] = (__bf16)(0.002f * (float)(lane - e));
    }
    floatx16 c0 = {}, c1 = {};
    float x[K > 0 ? K : 1], y[E > 0 ? E : 1];
#pragma unroll
    for (int i = 0; i < (K > 0 ? K : 1); ++i) x[i] = 1.0f + 1e-3f * (float)(lane + i);
#pragma unroll
    for (int i = 0; i < (E > 0 ? E : 1); ++i) y[i] = -1.0f - 1e-3f * (float)(lane + i);
    const float m = 0.999f, sm = 1e-6f;
    const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
      c0 = fa::mfma32(a, b, c0);
#pragma unroll
      for (int k = 0; k < K; ++k) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[k]) : "v"(m), "v"(sm));
#pragma unroll
      for (int e = 0; e < E; ++e) asm volatile("v_exp_f32 %0, %0" : "+v"(y[e]));
      c1 = fa::mfma32(b, a, c1);
#pragma unroll
      for (int k = 0; k < K; ++k) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[k]) : "v"(m), "v"(sm));
#pragma unroll
      for (int e = 0; e < E; ++e) asm volatile("v_exp_f32 %0, %0" : "+v"(y[e]));
    }
    t = __builtin_amdgcn_s_memtime() - t0;
    r = __builtin_amdgcn_s_memrealtime() - r0;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc += c0[q] + c1[q];
#pragma unroll
    for (int i = 0; i < (K > 0 ? K : 1); ++i) acc += x[i];
#pragma unroll
    for (int i = 0; i < (E > 0 ? E : 1); ++i) acc += y[i];
  } else if (valu_wave) {
    float x[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) x[i] = (E > 0 ? -1.0f : 1.0f) + 1e-3f * (float)(lane + i);
    const float m = 0.999f, sm = 1e-6f;
    const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
      if constexpr (E > 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) asm volatile("v_exp_f32 %0, %0" : "+v"(x[k]));
      } else {
#pragma unroll
        for (int k = 0; k < 12; ++k) asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[k]) : "v"(m), "v"(sm));
      }
    }
    t = __builtin_amdgcn_s_memtime() - t0;
    r = __builtin_amdgcn_s_memrealtime() - r0;
#pragma unroll
    for (int i = 0; i < 12; ++i) acc += x[i];
  }
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  out[gid] = acc;
  if (lane == 0) {
    ticks[2 * (gid / 64)] = t;
    ticks[2 * (gid / 64) + 1] = r;
  }
}

// Each wave runs `iters` rounds of four independent 32x32x16 bf16 MFMA chains on
// register operands and stores its accumulators once (so the chains are not removed).
__global__ __launch_bounds__(256, 2) void mfma_probe(float* __restrict__ out, int iters) {
  using fa::bf16x8;
  using fa::floatx16;
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)(lane + e));
    b[e] = (__bf16)(0.002f * (float)(lane - e));
  }
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = fa::mfma32(a, b, c0);
    c1 = fa::mfma32(b, a, c1);
    c2 = fa::mfma32(a, a, c2);
    c3 = fa::mfma32(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// LDS probe: every wave of 4-wave workgroups (64 KiB of LDS each, two per compute unit)
// runs `iters` rounds of eight LDS accesses of one kind at consecutive per-lane addresses
// (no bank conflicts) and folds what it reads into one word per thread. M: 0 ds_read_b128,
// 1 ds_read_b64, 2 ds_read_b64_tr_b16, 3 ds_read_b32, 4 ds_write_b128 (a wait for the
// writes ends each round). Each wave times its loop as the issue probe does.
template <int M>
__global__ __launch_bounds__(256, 2) void lds_probe(unsigned* __restrict__ out, long long* __restrict__ ticks,
                                                    int iters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 65536 / 4; i += 256) reinterpret_cast<unsigned*>(lds)[i] = (unsigned)i * 2654435761u;
  __syncthreads();
  constexpr int W = M == 0 || M == 4 ? 16 : M == 3 ? 4 : 8;  // bytes per lane
  // base < 32768; a round touches base ^ (0..240) + k * 2048 + W for k < 8: below 48 KiB
  const int base = (wave * 8192 + lane * W) & 32767;
  unsigned acc = 0;
  fa::u32x4 v4 = {(unsigned)lane, (unsigned)wave, 3u, 4u};
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    const int b = base ^ ((it & 15) << 4);
    if constexpr (M == 0) {
      fa::u32x4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const fa::u32x4*>(lds + b + k * 2048);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][3];
    } else if constexpr (M == 1) {
      fa::u32x2 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const fa::u32x2*>(lds + b + k * 2048);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][1];
    } else if constexpr (M == 2) {
      fa::i16x4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(fa::i16x4, lds + b + k * 2048));
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= __builtin_bit_cast(fa::u32x2, v[k])[0] ^ __builtin_bit_cast(fa::u32x2, v[k])[1];
    } else if constexpr (M == 3) {
      unsigned v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const unsigned*>(lds + b + k * 2048);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= v[k];
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) *reinterpret_cast<fa::u32x4*>(lds + b + k * 2048) = v4;
      v4[2] += 1u;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the round's writes are done
    }
  }
  const long long t = __builtin_amdgcn_s_memtime() - t0, r = __builtin_amdgcn_s_memrealtime() - r0;
  __syncthreads();
  if constexpr (M == 4) acc = reinterpret_cast<const unsigned*>(lds)[threadIdx.x * 16];
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  out[gid] = acc;
  if (lane == 0) {
    ticks[2 * (gid / 64)] = t;
    ticks[2 * (gid / 64) + 1] = r;
  }
}

// Tile probe: a model of the forward kernel's steady-state tile body with the same
// instruction mix and none of its data dependences. 4-wave workgroups (64 KiB of LDS, two
// per compute unit); per tile and wave, 32 MFMA slots: slots 0-15 accumulate into four
// chains (the P V half, A operand read by two ds_read_b64_tr_b16), slots 16-31 into two
// chains restarted from zero each tile (the Q K^T half, A operand one ds_read_b128); the
// operand reads run three slots ahead; NF independent v_fma_f32 and 33 independent
// v_exp_f32 are spread over the slots; one workgroup barrier per tile. With CP, each
// wave also issues the tile's K and V copies as the kernel does: after a wait for its
// earlier copies and the barrier, eight 1 KiB LDS-DMA loads into the LDS half the reads do
// not use, from a 256 KiB source that stays in the L2 cache.
constexpr int kTileProbeSrcBytes = 256 * 1024;
template <int NF, int CP>
__global__ __launch_bounds__(256, 2) void tile_probe(const unsigned char* __restrict__ src, float* __restrict__ out,
                                                     long long* __restrict__ ticks, int tiles) {
  using fa::bf16x8;
  using fa::floatx16;
  __shared__ __attribute__((aligned(16))) unsigned char lds[65536];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 65536 / 4; i += 256) reinterpret_cast<float*>(lds)[i] = 1e-3f * (float)(i & 255);
  __syncthreads();
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = (__bf16)(0.002f * (float)(lane - e));
  floatx16 c[4] = {}, d[2] = {};
  float x[12], y[4];
#pragma unroll
  for (int i = 0; i < 12; ++i) x[i] = 1.0f + 1e-3f * (float)(lane + i);
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = -1.0f - 1e-3f * (float)(lane + i);
  const float m = 0.999f, sm = 1e-6f;
  // operand reads: tb < 32768 and 16-byte aligned, slot offsets add at most 31 KiB + 512 + 16
  const int base = (wave * 4096 + lane * 16) & 32767;
  auto operand = [&](int tb, int s) {
    const int off = tb + (s & 31) * 1024;
    if (s % 32 >= 16) return *reinterpret_cast<const bf16x8*>(lds + off);
    const fa::i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(fa::i16x4, lds + off));
    const fa::i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(fa::i16x4, lds + off + 512));
    const fa::bf16x4 l = __builtin_bit_cast(fa::bf16x4, lo), h = __builtin_bit_cast(fa::bf16x4, hi);
    return bf16x8{l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  };
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(src), 0, kTileProbeSrcBytes, fa::kBufferWord3);
  const long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 q[4];
#pragma unroll
  for (int i = 0; i < 3; ++i) q[i] = operand(base, i);
  for (int t = 0; t < tiles; ++t) {
    if constexpr (CP) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      // LDS destination (t mod 2) * 32 KiB + (wave * 8 + i) KiB; source offset below 256 KiB
      unsigned char* stage = lds + 32768 * (t & 1);
      const int so = ((blockIdx.x * 7 + t) & 7) * 32768 + wave * 8192 + lane * 16;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, stage + (wave * 8 + i) * 1024), 16, so + i * 1024, 0, 0, 0);
    } else {
      __syncthreads();
    }
    const int tb = base ^ ((t & 7) << 4);
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      q[(s + 3) & 3] = operand(tb, s + 3);
      if (s < 16) c[s & 3] = fa::mfma32(q[s & 3], b, c[s & 3]);
      else d[s & 1] = fa::mfma32(q[s & 3], b, s < 18 ? floatx16{} : d[s & 1]);
#pragma unroll
      for (int k = 0; k < NF / 32 + (s < NF % 32 ? 1 : 0); ++k)
        asm volatile("v_fma_f32 %0, %0, %1, %2" : "+v"(x[(s * 4 + k) % 12]) : "v"(m), "v"(sm));
      asm volatile("v_exp_f32 %0, %0" : "+v"(y[s % 4]));
      if (s == 0) asm volatile("v_exp_f32 %0, %0" : "+v"(y[1]));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  const long long t = __builtin_amdgcn_s_memtime() - t0, r = __builtin_amdgcn_s_memrealtime() - r0;
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += c[0][i] + c[1][i] + c[2][i] + c[3][i] + d[0][i] + d[1][i];
#pragma unroll
  for (int i = 0; i < 12; ++i) acc += x[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc += y[i] + (float)q[i][0];
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  out[gid] = acc;
  if (lane == 0) {
    ticks[2 * (gid / 64)] = t;
    ticks[2 * (gid / 64) + 1] = r;
  }
}

// The calling thread's launch timer: a grow-only pool of event pairs (created on the device
// current when armed, kept until the process ends), how many are armed, and how many of
// those the main-kernel launches have taken.
struct LaunchTimer {
  std::vector<hipEvent_t> ev;  // start, stop, start, stop, ...
  int dev = -1;                // the device the events belong to
  int armed = 0;
  int taken = 0;
};
thread_local LaunchTimer t_timer;

}  // namespace

fa::LaunchEvents fa::next_launch_events() {
  LaunchTimer& t = t_timer;
  if (t.taken >= t.armed) return {nullptr, nullptr};
  const int i = t.taken++;
  return {t.ev[2 * i], t.ev[2 * i + 1]};
}

extern "C" {

int fa_probe_timer_arm(int n) {
  LaunchTimer& t = t_timer;
  if (n < 0 || n > FA_PROBE_TIMER_MAX) return FA_ERR_NULL;
  t.armed = t.taken = 0;
  if (n == 0) return FA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_DEVICE;
  if (dev != t.dev) {  // events of another device: start a new pool on this one
    for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
    t.ev.clear();
    t.dev = dev;
  }
  while ((int)t.ev.size() < 2 * n) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return FA_ERR_DEVICE;
    t.ev.push_back(e);
  }
  t.armed = n;
  t.taken = 0;
  return FA_OK;
}

int fa_probe_timer_read(float* us, int n) {
  LaunchTimer& t = t_timer;
  if (!us || n < 0 || n != t.taken) return FA_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess)
      return FA_ERR_DEVICE;
    us[i] = ms * 1000.f;
  }
  t.armed = t.taken = 0;
  return FA_OK;
}

int fa_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
    return FA_ERR_NULL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return FA_ERR_DEVICE;
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + 255) / 256;
  const int grid = (int)(want < (int64_t)cus * 16 ? want : (int64_t)cus * 16);
  hipLaunchKernelGGL(copy_probe, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const fa::u32x4*>(src), static_cast<fa::u32x4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_probe_read(const void* src, int64_t bytes, unsigned* sink, int sink_words, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0) return FA_ERR_NULL;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return FA_ERR_DEVICE;
  const int64_t n16 = bytes / 16;
  const int64_t want = (n16 + 255) / 256;
  const int grid = (int)(want < (int64_t)cus * 16 ? want : (int64_t)cus * 16);
  if (sink_words < grid) return FA_ERR_SHAPE;
  hipLaunchKernelGGL(read_probe, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const fa::u32x4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_probe_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return FA_ERR_NULL;
  hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_probe_issue(int role, int valu_ops, int exps, int blocks, int iters, float* out, long long* ticks,
                   void* stream) {
  if (!out || !ticks || blocks <= 0 || iters <= 0 || role < 0 || role > 4) return FA_ERR_NULL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(blocks), block(role == 0 ? 256 : 512);
#define FA_ISSUE(R, K, E) hipLaunchKernelGGL((issue_probe<R, K, E>), grid, block, 0, st, out, ticks, iters)
  if (role == 0) {
    const int key = valu_ops * 8 + exps;
    switch (key) {
      case 0 * 8 + 0: FA_ISSUE(0, 0, 0); break;
      case 2 * 8 + 0: FA_ISSUE(0, 2, 0); break;
      case 4 * 8 + 0: FA_ISSUE(0, 4, 0); break;
      case 6 * 8 + 0: FA_ISSUE(0, 6, 0); break;
      case 8 * 8 + 0: FA_ISSUE(0, 8, 0); break;
      case 12 * 8 + 0: FA_ISSUE(0, 12, 0); break;
      case 0 * 8 + 1: FA_ISSUE(0, 0, 1); break;
      case 0 * 8 + 2: FA_ISSUE(0, 0, 2); break;
      case 0 * 8 + 4: FA_ISSUE(0, 0, 4); break;
      case 4 * 8 + 1: FA_ISSUE(0, 4, 1); break;
      case 4 * 8 + 2: FA_ISSUE(0, 4, 2); break;
      default: return FA_ERR_SHAPE;
    }
  } else {
    if (valu_ops != 0) return FA_ERR_SHAPE;
    const bool e = exps > 0;
    switch (role) {
      case 1: if (e) FA_ISSUE(1, 0, 1); else FA_ISSUE(1, 0, 0); break;
      case 2: if (e) FA_ISSUE(2, 0, 1); else FA_ISSUE(2, 0, 0); break;
      case 3: if (e) FA_ISSUE(3, 0, 1); else FA_ISSUE(3, 0, 0); break;
      default: if (e) FA_ISSUE(4, 0, 1); else FA_ISSUE(4, 0, 0); break;
    }
  }
#undef FA_ISSUE
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_probe_lds(int mode, int blocks, int iters, unsigned* out, long long* ticks, void* stream) {
  if (!out || !ticks || blocks <= 0 || iters <= 0) return FA_ERR_NULL;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(lds_probe<0>, dim3(blocks), dim3(256), 0, st, out, ticks, iters); break;
    case 1: hipLaunchKernelGGL(lds_probe<1>, dim3(blocks), dim3(256), 0, st, out, ticks, iters); break;
    case 2: hipLaunchKernelGGL(lds_probe<2>, dim3(blocks), dim3(256), 0, st, out, ticks, iters); break;
    case 3: hipLaunchKernelGGL(lds_probe<3>, dim3(blocks), dim3(256), 0, st, out, ticks, iters); break;
    case 4: hipLaunchKernelGGL(lds_probe<4>, dim3(blocks), dim3(256), 0, st, out, ticks, iters); break;
    default: return FA_ERR_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_probe_tile(int copies, int valu_ops, int blocks, int tiles, const void* src, int64_t src_bytes, float* out,
                  long long* ticks, void* stream) {
  if (!out || !ticks || blocks <= 0 || tiles <= 0) return FA_ERR_NULL;
  if (copies && (!src || reinterpret_cast<uintptr_t>(src) % 16 != 0 || src_bytes < kTileProbeSrcBytes))
    return copies && !src ? FA_ERR_NULL : FA_ERR_SHAPE;
  if ((copies != 0 && copies != 1) || (valu_ops != 0 && valu_ops != 117)) return FA_ERR_SHAPE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const unsigned char* g = static_cast<const unsigned char*>(src);
  const dim3 grid(blocks), block(256);
  if (valu_ops == 117) {
    if (copies) hipLaunchKernelGGL((tile_probe<117, 1>), grid, block, 0, st, g, out, ticks, tiles);
    else hipLaunchKernelGGL((tile_probe<117, 0>), grid, block, 0, st, g, out, ticks, tiles);
  } else {
    if (copies) hipLaunchKernelGGL((tile_probe<0, 1>), grid, block, 0, st, g, out, ticks, tiles);
    else hipLaunchKernelGGL((tile_probe<0, 0>), grid, block, 0, st, g, out, ticks, tiles);
  }
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

double fa_probe_mfma_flops(int blocks, int iters) {
  // four waves per block, four MFMAs per round, 2 * 32 * 32 * 16 FLOP each
  return (double)blocks * 4.0 * (double)iters * 4.0 * 32768.0;
}

}  // extern "C"

// Device helpers for the gfx950 verification kernels: row addressing,
// 16-byte vector loads, wave64 / work-group reductions and scans, the
// counter-based SplitMix64 uniform, and the completion tickets that let the
// last work-group of a request finish it.
//
// Completion tickets without device-scope fences.  On this part a
// device-scope release (an L2 write-back) inside a streaming kernel costs
// about 1 us per work-group per XCD, so no kernel here uses one.  Instead a
// work-group publishes its partial result with device-scope relaxed atomic
// stores, which compile to stores with the sc1 bit: written through to the
// device coherence point, past the XCD's L2.  It then waits until those
// stores have completed (s_waitcnt vmcnt(0)) and only then increments the
// request's counter with a device-scope atomic.  The work-group that
// receives the last ticket reads the partials with device-scope relaxed
// atomic loads (sc1: served from the coherence point, not from a stale L2
// line).  Every partial was complete before its ticket was taken, and the
// last ticket is taken after every other ticket, so the reader sees them all.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace specv {

// ---------------------------------------------------------------------------
// Coherent publication and completion tickets
// ---------------------------------------------------------------------------

__device__ __forceinline__ void st_dev(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_d(double* p, double v) {
  st_dev(reinterpret_cast<uint64_t*>(p), static_cast<uint64_t>(__double_as_longlong(v)));
}
__device__ __forceinline__ double ld_dev_d(const double* p) {
  return __longlong_as_double(static_cast<long long>(ld_dev(reinterpret_cast<const uint64_t*>(p))));
}
__device__ __forceinline__ uint64_t pack2(float a, float b) {
  return static_cast<uint64_t>(__float_as_uint(a)) |
         (static_cast<uint64_t>(__float_as_uint(b)) << 32);
}
__device__ __forceinline__ float unpack_lo(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v)); }
__device__ __forceinline__ float unpack_hi(uint64_t v) { return __uint_as_float(static_cast<uint32_t>(v >> 32)); }

__device__ __forceinline__ unsigned ld_dev_u32(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_dev_f(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev_f(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Polls of a bounded wait before it gives up (a few seconds; a legitimate
// wait lasts microseconds).
constexpr long kSpinLimit = 1L << 20;

// Wait until this wave's earlier stores have completed.
__device__ __forceinline__ void wait_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One thread per work-group calls this after its coherent stores.  Returns
// true for the last of `total` arrivals; that caller also resets the counter
// to zero for the next call.
__device__ __forceinline__ bool arrive(unsigned* counter, unsigned total) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores above are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const unsigned t = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool last = (t == total - 1u);
  if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// Work-group form: thread 0 arrives; the answer is broadcast.
__device__ __forceinline__ bool block_arrive(unsigned* counter, unsigned total) {
  __shared__ int s_last;
  if (threadIdx.x == 0) s_last = arrive(counter, total) ? 1 : 0;
  __syncthreads();
  return s_last != 0;
}

// Wave form (wave 0 of a work-group whose other waves have left): lane 0
// arrives; the answer is broadcast across the wave.
__device__ __forceinline__ bool wave_arrive(unsigned* counter, unsigned total) {
  int last = 0;
  if ((threadIdx.x & 63) == 0) last = arrive(counter, total) ? 1 : 0;
  return __shfl(last, 0, 64) != 0;
}

// Orders this wave's shared-memory writes before its later reads (lanes
// exchange values through shared memory without a work-group barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Elements per 16-byte vector for each input dtype (0 = f32, 1 = bf16).
template <int DT>
struct Elems {
  static constexpr int kVec = DT == 1 ? 8 : 4;
  static constexpr int kBytes = DT == 1 ? 2 : 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte non-temporal buffer loads from one row: the row's base address
// and size sit in a buffer resource (SGPRs), each load takes a per-lane
// 32-bit byte offset plus a uniform one, so the streaming loops need no
// 64-bit address arithmetic per load.  Rows must be shorter than 2 GiB.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit buffer, gfx9 family
// Cache policy of the row sweeps' loads (tunable at build time): nt, i.e.
// streamed data that is read once.
#ifndef SPEC_ROW_LOAD_POLICY
#define SPEC_ROW_LOAD_POLICY 2
#endif
constexpr int kLoadNonTemporal = SPEC_ROW_LOAD_POLICY;

struct RowBuf {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ RowBuf(const void* base, uint32_t bytes)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                               kBufferWord3)) {}
  __device__ __forceinline__ u32x4 load_nt(uint32_t lane_off, uint32_t uniform_off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)lane_off, (int)uniform_off,
                                                 kLoadNonTemporal);
  }
};

// The Elems<DT>::kVec elements of one 16-byte word as floats.
template <int DT>
__device__ __forceinline__ void unpack16(const u32x4& w, float* x) {
  if constexpr (DT == 1) {
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
}

// One element of a row as float.
template <int DT>
__device__ __forceinline__ float load_elem(const void* row, long j) {
  if constexpr (DT == 1) {
    const uint16_t h = reinterpret_cast<const uint16_t*>(row)[j];
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  } else {
    return reinterpret_cast<const float*>(row)[j];
  }
}

// NE elements starting at element index e0 (NE == Elems<DT>::kVec: one
// 16-byte load that must be 16-byte aligned; NE == 1: one scalar load).
// NT: non-temporal load (streamed data that is read once).
template <int DT, int NE, bool NT = false>
__device__ __forceinline__ void load_group(const void* row, long e0, float (&x)[NE]) {
  if constexpr (NE == 1) {
    x[0] = load_elem<DT>(row, e0);
  } else {
    static_assert(NE == Elems<DT>::kVec, "vector group must be 16 bytes");
    const u32x4* ptr = reinterpret_cast<const u32x4*>(
        reinterpret_cast<const char*>(row) + e0 * Elems<DT>::kBytes);
    const u32x4 w = NT ? __builtin_nontemporal_load(ptr) : *ptr;
    if constexpr (DT == 1) {
      x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
      x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
      x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
      x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    } else {
      x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
      x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
  }
}

// ---------------------------------------------------------------------------
// Wave64 shuffles
// ---------------------------------------------------------------------------

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ double shfl_up_d(double v, int d) { return __shfl_up(v, d, 64); }

// ---------------------------------------------------------------------------
// (max, sum of exp2((x - max) * c)) pairs: the streaming softmax statistic
// ---------------------------------------------------------------------------

// Float32 product rounded on its own.  The compiler's default contraction
// would fuse a plain `a * b` into a following add (and HIP's __fmul_rn is a
// plain multiply), giving fma(a, b, z): then fl(m c) - fl(m c) is no longer
// exactly 0 but the rounding error of m c, and merges that should leave a
// sum untouched scale it by 2^(that error) at every reduction level.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// Combine two (m, s) pairs, each s (float64) relative to 2^fl32(m c).
// -inf maxima (no finite element yet) carry s = 0.
__device__ __forceinline__ void ms_merge(float& m, double& s, float m2, double s2, float c) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  // Each s is relative to exactly the rounded product fl32(m c); the side
  // that holds the new maximum keeps a factor of exactly 1.
  const float mn = fmaxf(m, m2);
  const float mcn = mul_rn(mn, c);
  s = s * (double)__builtin_amdgcn_exp2f(mul_rn(m, c) - mcn) +
      s2 * (double)__builtin_amdgcn_exp2f(mul_rn(m2, c) - mcn);
  m = mn;
}

// Wave reduction of (m, s); the result is valid in every lane.
__device__ __forceinline__ void wave_reduce_ms(float& m, double& s, float c) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = shfl_xor_f(m, o);
    const double s2 = shfl_xor_d(s, o);
    ms_merge(m, s, m2, s2, c);
  }
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_d(v, o);
  return v;
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ double wave_inclusive_scan_d(double v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = shfl_up_d(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Exclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ double wave_exclusive_scan_d(double v) {
  const int lane = threadIdx.x & 63;
  double inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = shfl_up_d(inc, d);
    if (lane >= d) inc += o;
  }
  return inc - v;
}

// Work-group reduction of (m, s); result valid in thread 0.
__device__ __forceinline__ void block_reduce_ms(float& m, double& s, float c) {
  __shared__ float sm[kWaves];
  __shared__ double ss[kWaves];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = shfl_xor_f(m, o);
    const double s2 = shfl_xor_d(s, o);
    ms_merge(m, s, m2, s2, c);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) { sm[wave] = m; ss[wave] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    m = sm[0]; s = ss[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) ms_merge(m, s, sm[w], ss[w], c);
  }
}

// ---------------------------------------------------------------------------
// (value, index) argmax with lowest index on ties
// ---------------------------------------------------------------------------

__device__ __forceinline__ void am_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

// Work-group argmax; result valid in thread 0.
__device__ __forceinline__ void block_reduce_am(float& v, int& i) {
  __shared__ float sv[kWaves];
  __shared__ int si[kWaves];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = shfl_xor_f(v, o);
    const int i2 = shfl_xor_i(i, o);
    am_merge(v, i, v2, i2);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) { sv[wave] = v; si[wave] = i; }
  __syncthreads();
  if (threadIdx.x == 0) {
    v = sv[0]; i = si[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) am_merge(v, i, sv[w], si[w]);
  }
}

// ---------------------------------------------------------------------------
// float64 sums and scans over a work-group
// ---------------------------------------------------------------------------

// Sum over the work-group (fixed order); result broadcast to all threads.
__device__ __forceinline__ double block_sum_d(double v) {
  __shared__ double sd[kWaves];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_d(v, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sd[wave] = v;
  __syncthreads();
  double t = sd[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t += sd[w];
  return t;
}

// Sums of N doubles per thread over the work-group, in place (every thread
// receives the totals).
template <int N>
__device__ __forceinline__ void block_sum_dn(double (&v)[N]) {
  __shared__ double sd[kWaves][N];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int q = 0; q < N; ++q) v[q] += shfl_xor_d(v[q], o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < N; ++q) sd[wave][q] = v[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < N; ++q) {
    double t = sd[0][q];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += sd[w][q];
    v[q] = t;
  }
}

// Sums of five doubles per thread over the work-group, in place (every
// thread receives the totals).
__device__ __forceinline__ void block_sum_d5(double (&v)[5]) {
  __shared__ double sd[kWaves][5];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int q = 0; q < 5; ++q) v[q] += shfl_xor_d(v[q], o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int q = 0; q < 5; ++q) sd[wave][q] = v[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    double t = sd[0][q];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += sd[w][q];
    v[q] = t;
  }
}

// Exclusive scan of one double per thread across the work-group.
// Returns the exclusive prefix for this thread.
__device__ __forceinline__ double block_exclusive_scan_d(double v) {
  __shared__ double wsum[kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const double o = shfl_up_d(inc, d);
    if (lane >= d) inc += o;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  return base + (inc - v);
}

// Exclusive prefix sums of N values over the work-group, and their
// work-group totals (every thread receives them).
template <int N>
__device__ __forceinline__ void block_exclusive_scan_total_dn(const double (&v)[N],
                                                              double (&excl)[N],
                                                              double (&total)[N]) {
  __shared__ double wsum[N][kWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double inc[N];
#pragma unroll
  for (int j = 0; j < N; ++j) inc[j] = v[j];
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const double o = shfl_up_d(inc[j], d);
      if (lane >= d) inc[j] += o;
    }
  }
  __syncthreads();
  if (lane == 63) {
#pragma unroll
    for (int j = 0; j < N; ++j) wsum[j][wave] = inc[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < N; ++j) {
    double base = 0.0, all = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (w < wave) base += wsum[j][w];
      all += wsum[j][w];
    }
    excl[j] = base + (inc[j] - v[j]);
    total[j] = all;
  }
}

// Minimum of an int over the work-group, broadcast.
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int block_min_i(int v) {
  __shared__ int si[kWaves];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, shfl_xor_i(v, o));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) si[wave] = v;
  __syncthreads();
  int t = si[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) t = min(t, si[w]);
  return t;
}

// ---------------------------------------------------------------------------
// SplitMix64 uniform (Steele, Lea & Flood 2014), counter form
// ---------------------------------------------------------------------------

__device__ __forceinline__ float splitmix_uniform(uint64_t seed, uint64_t ctr) {
  uint64_t z = seed + (ctr + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z = z ^ (z >> 31);
  return static_cast<float>(static_cast<uint32_t>(z >> 40)) * 0x1.0p-24f;
}

// Uniform for (request b, position i, slot) from an array or from the seed.
__device__ __forceinline__ float get_uniform(const float* u, uint64_t seed, uint64_t ctr0,
                                             int b, int i, int slot, int k) {
  const long idx = ((long)b * (k + 1) + i) * 2 + slot;
  if (u != nullptr) return u[idx];
  return splitmix_uniform(seed, ctr0 + (uint64_t)idx);
}

}  // namespace specv
